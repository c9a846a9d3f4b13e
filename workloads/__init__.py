"""Seeded synthetic inputs for paged varlen attention.

This module is shared by the tests, the benchmark and the smoke check.  It holds
bookkeeping and random draws only -- sequence lengths, block allocation, the
block table, slot numbers, and N(0, 1) tensors -- and none of the attention or
store arithmetic.  Both the CPU oracle and the HIP path consume what it returns;
neither is imported here.

Conventions (they follow the serving bookkeeping the pages describe):

* ``q_lens[b]``  -- new query tokens of sequence b (the extend length).
* ``k_lens[b]``  -- all key tokens of sequence b so far, cached prefix plus the
  new tokens (the device length); the cached prefix is ``k_lens - q_lens``.
  [장부가 커널 인자로 바뀌는 지점과 CUDA graph, section "장부에서 텐서로"]
* The KV pool is ``[num_blocks, 16, Hkv, D]``; token ``t`` of sequence ``b`` lives
  in physical block ``block_table[b, t // 16]`` at row ``t % 16``; its slot number is
  ``block * 16 + row``.  [Transformer 추론 커널 (3/10), §14; tiny-vLLM series,
  entry 6 (16-token blocks)]
* Physical blocks are handed out from a seeded permutation of the pool, in
  (sequence, logical block) order, so neighbouring logical blocks are scattered.
* Pool blocks nobody owns, tail rows of partial last blocks, and table entries
  past a sequence's last block are "poison": NaN data, and the table entries
  point at a NaN-filled block that no sequence owns.

Random draws, in this order from ``numpy.random.default_rng(seed)``: lengths
(inclusive bounds), the block permutation, Q, K, V (float32 standard normal).
bf16 inputs are the float32 draws rounded to nearest-even by torch on the CPU.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

BLOCK_SIZE = 16


@dataclass
class PagedBatch:
    """One varlen batch over a paged KV pool (host arrays)."""

    dtype: str                 # "fp32" or "bf16"
    Hq: int
    Hkv: int
    D: int
    scale: float
    causal: bool
    q_lens: np.ndarray         # int32 [B]
    k_lens: np.ndarray         # int32 [B]   (= seqlens_k)
    cu_seqlens_q: np.ndarray   # int32 [B+1]
    cu_seqlens_k: np.ndarray   # int32 [B+1] offsets of each sequence's rows in k_tokens
    block_table: np.ndarray    # int32 [B, MB]
    num_blocks: int            # NB, pool size in blocks
    poison_block: int          # an unowned block id; unused table entries point here
    q: np.ndarray              # float32 [T, Hq, D] (bf16-representable when dtype == "bf16")
    k_tokens: np.ndarray       # float32 [sum k_lens, Hkv, D], sequence-major, position order
    v_tokens: np.ndarray       # float32 [sum k_lens, Hkv, D]
    slots: np.ndarray          # int32 [sum k_lens], slot of every key token
    name: str = ""
    meta: dict = field(default_factory=dict)
    window: int = 0            # sliding window (causal only): row at position p sees keys p-window+1 .. p; 0 = none

    # ---- derived views -------------------------------------------------
    @property
    def B(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def T(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def MB(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def cached_lens(self) -> np.ndarray:
        return (self.k_lens - self.q_lens).astype(np.int32)

    def new_token_rows(self) -> np.ndarray:
        """Indices into k_tokens of the new tokens (the last q_lens[b] of each sequence)."""
        idx = []
        for b in range(self.B):
            s, e = int(self.cu_seqlens_k[b]), int(self.cu_seqlens_k[b + 1])
            idx.append(np.arange(e - int(self.q_lens[b]), e))
        return np.concatenate(idx) if idx else np.zeros(0, np.int64)

    def cached_token_rows(self) -> np.ndarray:
        idx = []
        for b in range(self.B):
            s, e = int(self.cu_seqlens_k[b]), int(self.cu_seqlens_k[b + 1])
            idx.append(np.arange(s, e - int(self.q_lens[b])))
        return np.concatenate(idx) if idx else np.zeros(0, np.int64)

    def store_rows(self) -> np.ndarray:
        """Indices into k_tokens/slots that write each slot exactly once (rows of
        a shared prefix appear in several sequences but own one slot)."""
        _, first = np.unique(self.slots, return_index=True)
        return np.sort(first)

    def pool_shape(self):
        return (self.num_blocks, BLOCK_SIZE, self.Hkv, self.D)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bf16 -> float32 (exact), via torch on the CPU."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def make_batch(
    seed: int,
    q_lens: Sequence[int] | None = None,
    k_lens: Sequence[int] | None = None,
    *,
    Hq: int,
    Hkv: int,
    D: int,
    dtype: str = "bf16",
    causal: bool = True,
    scale: Optional[float] = None,
    extra_blocks: int = 4,
    extra_table_cols: int = 0,
    len_draw=None,
    name: str = "",
    shared_prefix_blocks: int = 0,
    window: int = 0,
) -> PagedBatch:
    """Draw one batch.

    Either pass ``q_lens``/``k_lens`` explicitly, or pass ``len_draw(rng) ->
    (q_lens, k_lens)`` so the lengths come from the same seeded stream first.
    ``shared_prefix_blocks`` > 0 makes every sequence reuse sequence 0's first
    physical blocks (a shared prefix: several table rows name the same blocks);
    the shared K/V rows are then identical across those sequences.
    """
    if dtype not in ("fp32", "bf16"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    if len_draw is not None:
        q_lens, k_lens = len_draw(rng)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    k_lens = np.asarray(k_lens, dtype=np.int64)
    B = q_lens.shape[0]
    if k_lens.shape != (B,) or B < 1:
        raise ValueError("q_lens and k_lens must be equal-length, non-empty")
    if np.any(q_lens < 1) or np.any(k_lens < q_lens):
        raise ValueError("need 1 <= q_len <= k_len for every sequence")

    nblk = (k_lens + BLOCK_SIZE - 1) // BLOCK_SIZE
    MB = int(nblk.max()) + int(extra_table_cols)
    if shared_prefix_blocks:
        sp = int(shared_prefix_blocks)
        if np.any(nblk < sp) or np.any(k_lens - q_lens < sp * BLOCK_SIZE):
            raise ValueError("shared prefix must lie inside every cached prefix")
        owned = int(nblk[0] + (nblk[1:] - sp).sum())
    else:
        sp = 0
        owned = int(nblk.sum())
    NB = owned + 1 + int(extra_blocks)  # +1: the poison block
    perm = rng.permutation(NB).astype(np.int64)
    poison = int(perm[owned])

    table = np.full((B, MB), poison, dtype=np.int64)
    nxt = 0
    for b in range(B):
        for j in range(int(nblk[b])):
            if sp and b > 0 and j < sp:
                table[b, j] = table[0, j]
            else:
                table[b, j] = perm[nxt]
                nxt += 1
    assert nxt == owned

    T = int(q_lens.sum())
    Ktot = int(k_lens.sum())
    q = rng.standard_normal((T, Hq, D), dtype=np.float32)
    k_tok = rng.standard_normal((Ktot, Hkv, D), dtype=np.float32)
    v_tok = rng.standard_normal((Ktot, Hkv, D), dtype=np.float32)

    cu_q = np.zeros(B + 1, np.int64)
    cu_q[1:] = np.cumsum(q_lens)
    cu_k = np.zeros(B + 1, np.int64)
    cu_k[1:] = np.cumsum(k_lens)

    if sp:
        # shared prefix tokens carry sequence 0's rows
        n = sp * BLOCK_SIZE
        for b in range(1, B):
            k_tok[cu_k[b]:cu_k[b] + n] = k_tok[0:n]
            v_tok[cu_k[b]:cu_k[b] + n] = v_tok[0:n]

    slots = np.empty(Ktot, np.int64)
    for b in range(B):
        pos = np.arange(int(k_lens[b]))
        slots[cu_k[b]:cu_k[b + 1]] = table[b, pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE

    if dtype == "bf16":
        q, k_tok, v_tok = round_to_bf16(q), round_to_bf16(k_tok), round_to_bf16(v_tok)
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    return PagedBatch(
        dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, scale=float(scale), causal=bool(causal),
        q_lens=q_lens.astype(np.int32), k_lens=k_lens.astype(np.int32),
        cu_seqlens_q=cu_q.astype(np.int32), cu_seqlens_k=cu_k.astype(np.int32),
        block_table=table.astype(np.int32), num_blocks=NB, poison_block=poison,
        q=q, k_tokens=k_tok, v_tokens=v_tok, slots=slots.astype(np.int32), name=name,
        window=int(window),
    )


# ---------------------------------------------------------------------------
# The five named workloads.  Shapes follow the sizes the pages use as examples:
# a 17-token prompt, 64 decode sequences with 32 query / 8 KV heads over
# 16-token pages, 16 x 512 prefill rows (M = 8192), and a 32K-token prompt.
# ---------------------------------------------------------------------------

def tiny_varlen_fp32(seed: int = 1) -> PagedBatch:
    """2 sequences of 17 and 9 prompt tokens, no cache, Hq 4 / Hkv 2, D 64, fp32."""
    return make_batch(seed, [17, 9], [17, 9], Hq=4, Hkv=2, D=64, dtype="fp32",
                      causal=True, extra_blocks=4, name="tiny_varlen_fp32")


def paged_decode_bf16(seed: int = 2, B: int = 64, lo: int = 128, hi: int = 2048,
                      Hq: int = 32, Hkv: int = 8, D: int = 64) -> PagedBatch:
    """B decode rows, context lengths uniform in [lo, hi] (the new token included)."""
    def draw(rng):
        k = rng.integers(lo, hi + 1, size=B)
        return np.ones(B, np.int64), k
    return make_batch(seed, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", causal=True,
                      len_draw=draw, name="paged_decode_bf16")


def causal_prefill_bf16(seed: int = 3, B: int = 16, L: int = 512) -> PagedBatch:
    return make_batch(seed, [L] * B, [L] * B, Hq=32, Hkv=8, D=128, dtype="bf16",
                      causal=True, name="causal_prefill_bf16")


def extend_prefill_bf16(seed: int = 4, B: int = 8, cmax: int = 4096,
                        elo: int = 512, ehi: int = 2048) -> PagedBatch:
    def draw(rng):
        c = rng.integers(0, cmax + 1, size=B)
        e = rng.integers(elo, ehi + 1, size=B)
        return e, c + e
    return make_batch(seed, Hq=32, Hkv=8, D=128, dtype="bf16", causal=True,
                      len_draw=draw, name="extend_prefill_bf16")


def long_prefill_bf16(seed: int = 5, L: int = 32768) -> PagedBatch:
    return make_batch(seed, [L], [L], Hq=32, Hkv=8, D=128, dtype="bf16", causal=True,
                      extra_blocks=4, name="long_prefill_bf16")


def mixed_prefill_decode_bf16(seed: int = 6, n_prefill: int = 2, prefill_len: int = 256, n_decode: int = 30,
                              lo: int = 128, hi: int = 2048) -> PagedBatch:
    """One batch mixing both phases, as a serving step schedules them: n_prefill
    prompts of prefill_len new tokens (no cached prefix) and n_decode sequences
    with one new token each over contexts U{lo..hi} (the new token included);
    M = 2 x 256 + 30 x 1 = 542 query rows at the defaults.  Heads and D as the
    causal prefill workload (32 / 8, D 128)."""
    def draw(rng):
        k_dec = rng.integers(lo, hi + 1, size=n_decode)
        q = np.concatenate([np.full(n_prefill, prefill_len), np.ones(n_decode, np.int64)])
        k = np.concatenate([np.full(n_prefill, prefill_len), k_dec])
        return q, k
    return make_batch(seed, Hq=32, Hkv=8, D=128, dtype="bf16", causal=True, len_draw=draw,
                      name="mixed_prefill_decode_bf16")


def sliding_window_decode_bf16(seed: int = 7, window: int = 512) -> PagedBatch:
    """The paged decode workload (64 rows over contexts U{128..2048}, 32 / 8
    heads, D 64) under a sliding window of ``window`` keys."""
    b = paged_decode_bf16(seed=seed)
    b.window = int(window)
    b.name = "sliding_window_decode_bf16"
    return b


def sliding_window_prefill_bf16(seed: int = 8, B: int = 4, L: int = 4096, window: int = 1024) -> PagedBatch:
    """B prompts of L tokens (no cached prefix), 32 / 8 heads, D 128, under a
    sliding window of ``window`` keys: every row past the first ``window``
    positions sees exactly ``window`` keys."""
    return make_batch(seed, [L] * B, [L] * B, Hq=32, Hkv=8, D=128, dtype="bf16", causal=True,
                      window=window, name="sliding_window_prefill_bf16")


NAMED = {
    "tiny_varlen_fp32": tiny_varlen_fp32,
    "paged_decode_bf16": paged_decode_bf16,
    "causal_prefill_bf16": causal_prefill_bf16,
    "extend_prefill_bf16": extend_prefill_bf16,
    "long_prefill_bf16": long_prefill_bf16,
    "mixed_prefill_decode_bf16": mixed_prefill_decode_bf16,
    "sliding_window_decode_bf16": sliding_window_decode_bf16,
    "sliding_window_prefill_bf16": sliding_window_prefill_bf16,
}


def attention_flops(batch: PagedBatch) -> int:
    """Algorithmic FLOPs: 4*D per visible (query row, key) pair per query head
    (2*D for the score, 2*D for the weighted sum of V).  Masked pairs and the
    softmax's exp/max/rescale are not counted."""
    pairs = 0
    W = int(batch.window)
    for b in range(batch.B):
        lq, lk = int(batch.q_lens[b]), int(batch.k_lens[b])
        if W:
            pos = np.arange(lk - lq, lk, dtype=np.int64)   # row positions
            pairs += int(np.minimum(pos + 1, W).sum())
        elif batch.causal and lq > 1:
            c = lk - lq
            pairs += lq * c + lq * (lq + 1) // 2
        else:
            pairs += lq * lk
    return 4 * batch.D * batch.Hq * pairs


def kv_bytes(batch: PagedBatch) -> int:
    """K and V bytes that attention must read once: every key row some query row
    sees, of every KV head (with a window: keys from the first row's window start)."""
    esize = 2 if batch.dtype == "bf16" else 4
    keys = batch.k_lens.astype(np.int64)
    if batch.window:
        first = np.maximum(0, keys - batch.q_lens.astype(np.int64) - int(batch.window) + 1)
        keys = keys - first
    return int(2 * int(keys.sum()) * batch.Hkv * batch.D * esize)


def io_bytes(batch: PagedBatch) -> int:
    """Minimum bytes for one attention call: K+V once, q read, out written, lse (fp32)
    written, plus the int32 metadata."""
    esize = 2 if batch.dtype == "bf16" else 4
    qo = 2 * batch.T * batch.Hq * batch.D * esize
    lse = batch.T * batch.Hq * 4
    meta = 4 * (batch.B * batch.MB + 2 * batch.B + 1)
    return kv_bytes(batch) + qo + lse + meta
