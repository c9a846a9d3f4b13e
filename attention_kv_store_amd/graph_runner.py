"""Decode steps replayed from captured HIP graphs, with bucket padding.

The decode step (attn_decode_append_paged: store each sequence's new K/V
row, attend its query row over all its keys) is captured once per bucket
size into a HIP graph over static device buffers.  A step of B sequences
copies its inputs into the buffers of the smallest bucket >= B, fills the
rows past B with dummy sequences -- one key each, every table entry pointing
at a reserved cache block that no real sequence owns, so their stores land
there -- and replays that bucket's graph.  This is the serving-loop remedy
for launch overhead described in "장부가 커널 인자로 바뀌는 지점과 CUDA graph"
(the graph runner that pads a decode batch to a captured size and replays)
and in "Transformer 추론 커널 (3/10)", §21.

Only the library's own kernels run inside the graphs; the copies into the
static buffers are torch device copies issued outside the graph, on the same
stream.  The workspace of each bucket is zero-filled once before capture and
the library leaves its counters at zero, so replays need no clearing.
"""
from __future__ import annotations

from typing import Dict, Sequence

from . import attn_decode_append_paged, workspace_size


class DecodeGraphRunner:
    """Captured decode steps for a fixed cache and head layout.

    k_cache, v_cache: the [NB, 16, Hkv, D] pools (bf16 or fp32);
    reserved_block: a block index of the pool that no sequence uses (the
    dummy rows' table entries point at it and their new rows are stored there);
    buckets: batch sizes to capture (ascending); max_blocks: table width;
    Hq: query heads; scale: score scale; num_splits: 0 = automatic;
    window: sliding window of every captured step (0 = none), see
    attn_decode_append_paged.
    """

    def __init__(self, k_cache, v_cache, reserved_block: int, buckets: Sequence[int], max_blocks: int, Hq: int,
                 scale: float, num_splits: int = 0, window: int = 0):
        import torch

        if not buckets or list(buckets) != sorted(set(int(b) for b in buckets)) or buckets[0] < 1:
            raise ValueError("buckets must be distinct positive sizes in ascending order")
        if not 0 <= reserved_block < k_cache.shape[0]:
            raise ValueError("reserved_block must name a block of the pool")
        self.k_cache, self.v_cache = k_cache, v_cache
        self.reserved_block = int(reserved_block)
        self.buckets = [int(b) for b in buckets]
        self.max_blocks = int(max_blocks)
        self.scale = float(scale)
        self.window = int(window)
        Hkv, D = k_cache.shape[2], k_cache.shape[3]
        dt, dev = k_cache.dtype, k_cache.device
        self.graphs: Dict[int, torch.cuda.CUDAGraph] = {}
        self.bufs: Dict[int, dict] = {}
        for nb in self.buckets:
            b = {
                "q": torch.zeros(nb, Hq, D, dtype=dt, device=dev),
                "k_new": torch.zeros(nb, Hkv, D, dtype=dt, device=dev),
                "v_new": torch.zeros(nb, Hkv, D, dtype=dt, device=dev),
                "table": torch.full((nb, self.max_blocks), self.reserved_block, dtype=torch.int32, device=dev),
                "lens": torch.ones(nb, dtype=torch.int32, device=dev),
                "out": torch.zeros(nb, Hq, D, dtype=dt, device=dev),
                "lse": torch.zeros(nb, Hq, dtype=torch.float32, device=dev),
            }
            need = workspace_size(b["q"], k_cache, b["table"], num_splits=num_splits)
            b["ws"] = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
            self.bufs[nb] = b

            def step(b=b):
                attn_decode_append_paged(b["q"], b["k_new"], b["v_new"], k_cache, v_cache, b["table"], b["lens"],
                                         self.scale, out=b["out"], lse=b["lse"], num_splits=num_splits,
                                         workspace=b["ws"], window=self.window)

            step()   # warm-up outside the capture (first-call set-up of the library)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            self.graphs[nb] = g
        torch.cuda.synchronize()

    def bucket_for(self, B: int) -> int:
        for nb in self.buckets:
            if nb >= B:
                return nb
        raise ValueError(f"batch of {B} exceeds the largest captured bucket {self.buckets[-1]}")

    def step(self, q, k_new, v_new, block_table, seqlens_k):
        """One decode step for B <= max bucket sequences; returns views
        (out [B, Hq, D], lse [B, Hq]) of the bucket's output buffers, valid
        until the next step that uses the same bucket.  The dummy rows all
        store their (stale) new rows into row 0 of the reserved block; nothing
        reads it -- a dummy row's only key is its own new row, which the
        kernel takes from k_new -- so those colliding stores are harmless."""
        B = q.shape[0]
        nb = self.bucket_for(B)
        b = self.bufs[nb]
        if block_table.shape[1] > self.max_blocks:
            raise ValueError("block_table wider than the captured table")
        b["q"][:B].copy_(q)
        b["k_new"][:B].copy_(k_new)
        b["v_new"][:B].copy_(v_new)
        b["table"][:B, :block_table.shape[1]].copy_(block_table)
        b["table"][:B, block_table.shape[1]:].fill_(self.reserved_block)
        b["lens"][:B].copy_(seqlens_k)
        if B < nb:
            # dummy rows: one key each, in the reserved block
            b["table"][B:].fill_(self.reserved_block)
            b["lens"][B:].fill_(1)
        self.graphs[nb].replay()
        return b["out"][:B], b["lse"][:B]
