"""Plain-definition attention over a paged KV cache, numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix what is computed:

* O = softmax(Q K^T / sqrt(d) + mask) V  -- Transformer 추론 커널 (3/10), §10.
  The scale is an explicit argument here; 1/sqrt(D) is what the workloads pass.
* FlashAttention reaches that same result exactly, only on a different I/O
  schedule (same page, §11), so the materialised definition is the oracle.
* Paged address translation: logical position -> block_table[seq, pos // page]
  -> physical block, row pos % page  (same page, §14); page = 16 tokens
  (tiny-vLLM series, entry 6).
* GQA: several query heads share one KV head (same page, §15).  Reading: query
  head h uses KV head h // (Hq / Hkv).
* Causal with a cached prefix.  Reading: the new row i of a sequence with c
  cached tokens sits at position c + i and sees keys 0 .. c + i (bottom-right
  alignment); a one-row decode sees every key.  The lengths follow the serving
  bookkeeping (장부가 커널 인자로 바뀌는 지점과 CUDA graph, "장부에서 텐서로"):
  query length = extend length, key length = the whole length so far.
* lse (reading): natural log of the sum over visible keys of exp(scale q.k).
* Sliding window (reading).  The pages list it as one of the mask variants a
  kernel dispatch must cover and a test must exercise (Transformer 추론 커널
  (3/10), §19 and §24) without defining it.  Plain reading: with window W >= 1
  (causal only) the row at position p sees keys max(0, p - W + 1) .. p, the W
  most recent positions, its own included.  A one-row decode sits at position
  Lk - 1 and so sees the last W keys.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

BLOCK_SIZE = 16


def gather_sequence(cache: np.ndarray, table_row: np.ndarray, length: int,
                    block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Rows 0..length-1 of one sequence from a paged pool ``[NB, page, Hkv, D]``.

    Only the table entries that cover those rows are read.
    """
    t = np.arange(int(length))
    blocks = np.asarray(table_row, dtype=np.int64)[t // block_size]
    return cache[blocks, t % block_size]


def _validate(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, block_size):
    if q.ndim != 3 or k_cache.ndim != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [T, Hq, D] and caches [NB, page, Hkv, D]")
    T, Hq, D = q.shape
    NB, page, Hkv, Dk = k_cache.shape
    if page != block_size or Dk != D:
        raise ValueError("cache page size / head dim mismatch")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    B = seqlens_k.shape[0]
    if cu_seqlens_q.shape != (B + 1,) or block_table.ndim != 2 or block_table.shape[0] != B:
        raise ValueError("metadata shapes disagree")
    if cu_seqlens_q[0] != 0 or cu_seqlens_q[-1] != T or np.any(np.diff(cu_seqlens_q) < 1):
        raise ValueError("cu_seqlens_q must start at 0, end at T and strictly increase")
    lq = np.diff(cu_seqlens_q)
    if np.any(seqlens_k < lq):
        raise ValueError("every sequence needs k_len >= q_len")
    if np.any((seqlens_k + block_size - 1) // block_size > block_table.shape[1]):
        raise ValueError("block table too narrow")


def attention_oracle(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k,
                     scale: float, causal: bool, *, window: int = 0,
                     rows: Optional[Sequence[int]] = None, row_block: int = 2048,
                     block_size: int = BLOCK_SIZE):
    """Exact attention, float64.

    Arguments mirror the library call: ``q [T, Hq, D]``, ``k_cache``/``v_cache``
    ``[NB, 16, Hkv, D]``, ``block_table int [B, MB]``, ``cu_seqlens_q int [B+1]``,
    ``seqlens_k int [B]``.  Inputs of any float dtype are upcast to float64
    (exact for fp32 and bf16 values).

    ``window`` > 0 narrows the causal mask to the last ``window`` positions of
    each row (its own included); 0 means no window.

    ``rows`` optionally restricts the work to a subset of query tokens (global
    indices into q); rows are independent, so each is still the full definition.
    Returns ``(out [T, Hq, D], lse [T, Hq])``; rows not computed hold NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache)
    v_cache = np.asarray(v_cache)
    block_table = np.asarray(block_table, dtype=np.int64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    lk_all = np.asarray(seqlens_k, dtype=np.int64)
    _validate(q, k_cache, v_cache, block_table, cu, lk_all, block_size)
    window = int(window)
    if window < 0 or (window and not causal):
        raise ValueError("window must be >= 0, and a window needs the causal mask")
    T, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv

    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    want = None
    if rows is not None:
        want = np.zeros(T, dtype=bool)
        want[np.asarray(rows, dtype=np.int64)] = True

    for b in range(lk_all.shape[0]):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        sel = np.arange(r0, r1)
        if want is not None:
            sel = sel[want[r0:r1]]
            if sel.size == 0:
                continue
        lq, lk = r1 - r0, int(lk_all[b])
        cached = lk - lq
        Kb = gather_sequence(k_cache, block_table[b], lk, block_size).astype(np.float64)
        Vb = gather_sequence(v_cache, block_table[b], lk, block_size).astype(np.float64)
        for c0 in range(0, sel.size, row_block):
            rws = sel[c0:c0 + row_block]
            i = rws - r0                         # row index within the sequence
            # keys past the last visible one of this row block, and keys before
            # the window of its first row, are -inf for every row in it, so they
            # may be left out without changing anything
            ncols = lk if not (causal and lq > 1) else min(lk, cached + int(i.max()) + 1)
            k0 = max(0, cached + int(i.min()) - window + 1) if window else 0
            j = np.arange(k0, ncols)
            visible = np.ones((rws.size, ncols - k0), dtype=bool)
            if causal and lq > 1:
                visible = j[None, :] <= (cached + i)[:, None]
            if window:
                visible &= j[None, :] >= (cached + i - window + 1)[:, None]
            for h in range(Hq):
                g = h // G
                S = scale * (q[rws, h, :] @ Kb[k0:ncols, g, :].T)    # [rows, keys]
                S = np.where(visible, S, -np.inf)
                m = S.max(axis=1)
                P = np.exp(S - m[:, None])
                l = P.sum(axis=1)
                out[rws, h, :] = (P @ Vb[k0:ncols, g, :]) / l[:, None]
                lse[rws, h] = m + np.log(l)
    return out, lse


def lse_merge(parts):
    """Merge partial results over disjoint key sets of the same query rows.

    ``parts`` is a list of ``(out_i, lse_i)`` with ``out_i [..., D]`` normalised over
    its own keys and ``lse_i [...]``.  Following the pages' running-statistics
    update (Transformer 추론 커널 (3/10), §12: m_new = max(m, m_b) and
    l_new = e^(m - m_new) l + e^(m_b - m_new) l_b, the accumulator rescaled the
    same way) written in terms of lse = m + ln l:
        lse = M + ln sum_i exp(lse_i - M),  M = max_i lse_i
        out = sum_i exp(lse_i - lse) out_i
    Parts whose lse is -inf (no keys) carry weight 0 and are skipped.
    """
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    outs = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    M = lses.max(axis=0)
    w = np.where(np.isneginf(lses), 0.0, np.exp(lses - M[None]))
    s = w.sum(axis=0)
    lse = M + np.log(s)
    wn = w / s[None]
    out = np.zeros(outs.shape[1:])
    for i in range(outs.shape[0]):
        contrib = wn[i][..., None] * np.where(wn[i][..., None] == 0.0, 0.0, outs[i])
        out = out + contrib
    return out, lse
