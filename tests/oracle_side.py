"""Test helpers that run the CPU oracle on a workload batch (host only)."""
from __future__ import annotations

import numpy as np

from oracle import attention_oracle, kv_store_oracle
from workloads import BLOCK_SIZE, PagedBatch


def oracle_pool(batch: PagedBatch, dtype=np.float64):
    """The batch's paged pool as the oracle builds it: NaN everywhere, then every
    key token (cached prefix and new rows) scattered into its slot."""
    shape = batch.pool_shape()
    kc = np.full(shape, np.nan, dtype=dtype)
    vc = np.full(shape, np.nan, dtype=dtype)
    rows = batch.store_rows()
    return kv_store_oracle(batch.k_tokens[rows].astype(dtype), batch.v_tokens[rows].astype(dtype),
                           batch.slots[rows], kc, vc)


def oracle_attention(batch: PagedBatch, rows=None, pool=None, causal=None, window=None):
    kc, vc = pool if pool is not None else oracle_pool(batch)
    return attention_oracle(batch.q, kc, vc, batch.block_table, batch.cu_seqlens_q,
                            batch.k_lens, batch.scale,
                            batch.causal if causal is None else causal,
                            window=batch.window if window is None else window, rows=rows)


def gather_loop(cache, table_row, length):
    """Independent per-token gather written as a loop (for cross-checks)."""
    rows = []
    for t in range(length):
        rows.append(cache[int(table_row[t // BLOCK_SIZE]), t % BLOCK_SIZE])
    return np.stack(rows)
