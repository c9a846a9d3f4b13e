"""Device copies of the seeded workload batches (GPU side only).

Uploads a ``workloads.PagedBatch`` through torch and fills the paged pool with
the library's own ``kv_store_paged`` from the batch's token rows and slots.
Used by the benchmark and the GPU tests; it holds no attention arithmetic and
the CPU oracle never imports it.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import attention_kv_store_amd as kvs

from . import PagedBatch


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


def to_device_before_append(batch: PagedBatch, device="cuda", fill=float("nan")):
    """A decode batch (one new row per sequence) with only the cached prefix in
    the pool: the new tokens' slots keep ``fill``.  Returns ``(db, k_new, v_new)``
    with k_new / v_new [B, Hkv, D], the rows a fused append writes."""
    if batch.T != batch.B:
        raise ValueError("append needs one new row per sequence")
    dt = torch_dtype(batch)
    kc = torch.full(batch.pool_shape(), fill, dtype=dt, device=device)
    vc = torch.full(batch.pool_shape(), fill, dtype=dt, device=device)
    rows = np.intersect1d(batch.store_rows(), batch.cached_token_rows())
    if rows.size:
        kvs.kv_store_paged(torch.from_numpy(batch.k_tokens[rows]).to(dt).to(device),
                           torch.from_numpy(batch.v_tokens[rows]).to(dt).to(device),
                           torch.from_numpy(batch.slots[rows]).to(device), kc, vc)
    new = batch.new_token_rows()
    k_new = torch.from_numpy(batch.k_tokens[new]).to(dt).to(device)
    v_new = torch.from_numpy(batch.v_tokens[new]).to(dt).to(device)
    db = DeviceBatch(
        q=torch.from_numpy(batch.q).to(dt).to(device), k_cache=kc, v_cache=vc,
        block_table=torch.from_numpy(batch.block_table).to(device),
        cu_seqlens_q=torch.from_numpy(batch.cu_seqlens_q).to(device),
        seqlens_k=torch.from_numpy(batch.k_lens).to(device),
        scale=batch.scale, causal=batch.causal,
    )
    return db, k_new, v_new


def cache_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a device cache (uint16 for bf16, uint32 for fp32)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().view(np.uint32)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
