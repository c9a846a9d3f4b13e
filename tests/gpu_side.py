"""Test helpers that run a workload batch through the HIP library (GPU only).

The device pool is built by the library's own kv_store_paged from the batch's
token rows and slots; the oracle side builds its pool with the oracle store,
and the two pools are compared bitwise in the store test.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import attention_kv_store_amd as kvs
from workloads import PagedBatch


@dataclass
class DeviceBatch:
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    cu_seqlens_q: torch.Tensor
    seqlens_k: torch.Tensor
    scale: float
    causal: bool


def torch_dtype(batch: PagedBatch):
    return torch.bfloat16 if batch.dtype == "bf16" else torch.float32


def to_device(batch: PagedBatch, device="cuda", fill=float("nan")) -> DeviceBatch:
    dt = torch_dtype(batch)
    q = torch.from_numpy(batch.q).to(dt).to(device)
    kc = torch.full(batch.pool_shape(), fill, dtype=dt, device=device)
    vc = torch.full(batch.pool_shape(), fill, dtype=dt, device=device)
    rows = batch.store_rows()
    kt = torch.from_numpy(batch.k_tokens[rows]).to(dt).to(device)
    vt = torch.from_numpy(batch.v_tokens[rows]).to(dt).to(device)
    slots = torch.from_numpy(batch.slots[rows]).to(device)
    kvs.kv_store_paged(kt, vt, slots, kc, vc)
    return DeviceBatch(
        q=q, k_cache=kc, v_cache=vc,
        block_table=torch.from_numpy(batch.block_table).to(device),
        cu_seqlens_q=torch.from_numpy(batch.cu_seqlens_q).to(device),
        seqlens_k=torch.from_numpy(batch.k_lens).to(device),
        scale=batch.scale, causal=batch.causal,
    )


def run_attention(db: DeviceBatch, **kw):
    out, lse = kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q,
                                     db.seqlens_k, db.scale, db.causal, **kw)
    torch.cuda.synchronize()
    return out, lse


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
