"""Plain scatter of new K/V rows into a paged pool.  TEST INFRASTRUCTURE ONLY.

The pages put "RoPE + KV cache store" right before attention in a layer's step
list (Transformer 추론 커널 (3/10), §2), and the decode path appends the new
token's K/V to the cache (tiny-vLLM series, entry 5).  A slot number names one
token row of the pool; its page is slot // page_size and its row slot % page_size
(the token-granular table divided by page_size in 장부가 커널 인자로 바뀌는 지점과
CUDA graph, page-table part).  Reading: a negative slot means "skip this row".
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


def kv_store_oracle(k_new, v_new, slot_mapping, k_cache, v_cache, block_size: int = BLOCK_SIZE):
    """Return copies of ``k_cache``/``v_cache`` (``[NB, page, Hkv, D]``) with row
    ``t`` of ``k_new``/``v_new`` (``[T_new, Hkv, D]``) written at slot
    ``slot_mapping[t]`` for every non-negative slot.  Duplicate slots are invalid."""
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    if k_new.shape != v_new.shape or k_new.ndim != 3 or slots.shape != (k_new.shape[0],):
        raise ValueError("k_new/v_new must be [T, Hkv, D] with one slot per row")
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    if kc.shape[1] != block_size or kc.shape[2:] != k_new.shape[1:]:
        raise ValueError("pool shape mismatch")
    live = slots >= 0
    s = slots[live]
    if s.size and s.max() >= kc.shape[0] * block_size:
        raise ValueError("slot out of range")
    if np.unique(s).size != s.size:
        raise ValueError("duplicate slots")
    kc[s // block_size, s % block_size] = k_new[live]
    vc[s // block_size, s % block_size] = v_new[live]
    return kc, vc
