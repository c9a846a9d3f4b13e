"""Test helpers that run a workload batch through the HIP library (GPU only).

The device pool is built by the library's own kv_store_paged from the batch's
token rows and slots (workloads.device); the oracle side builds its pool with
the oracle store, and the two pools are compared bitwise in the store test.
"""
from __future__ import annotations

import torch

import attention_kv_store_amd as kvs
from workloads.device import (DeviceBatch, cache_bits, to_device, to_device_before_append,  # noqa: F401
                              to_f64, torch_dtype)


def run_append(db: DeviceBatch, k_new, v_new, **kw):
    out, lse = kvs.attn_decode_append_paged(db.q, k_new, v_new, db.k_cache, db.v_cache, db.block_table,
                                            db.seqlens_k, db.scale, **kw)
    torch.cuda.synchronize()
    return out, lse


def run_attention(db: DeviceBatch, **kw):
    out, lse = kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q,
                                     db.seqlens_k, db.scale, db.causal, **kw)
    torch.cuda.synchronize()
    return out, lse
