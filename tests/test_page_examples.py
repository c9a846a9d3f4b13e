"""Host bookkeeping against the numbers the pages print (tests/golden/page_examples.json)."""
from __future__ import annotations

import json
import os

import numpy as np

from workloads import BLOCK_SIZE, make_batch, tiny_varlen_fp32

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def test_prefill_rows():
    g = GOLD["prefill_rows"]
    b = make_batch(0, [g["prompt_tokens"]] * g["requests"], [g["prompt_tokens"]] * g["requests"],
                   Hq=2, Hkv=1, D=4, dtype="fp32")
    assert b.T == g["batch_tokens"]


def test_mixed_batch_tokens():
    g = GOLD["mixed_batch"]
    ql = [g["prefill_tokens_each"]] * g["prefill_requests"] + [1] * g["decode_requests"]
    kl = [g["prefill_tokens_each"]] * g["prefill_requests"] + [40] * g["decode_requests"]
    b = make_batch(0, ql, kl, Hq=2, Hkv=1, D=4, dtype="fp32")
    assert b.B == g["scheduled_requests"] and b.T == g["batch_tokens"]


def test_block_size_and_17_token_prompt():
    assert BLOCK_SIZE == GOLD["block_size"]["block_size"]
    n = GOLD["prompt_17"]["prompt_tokens"]
    b = make_batch(0, [n], [n], Hq=2, Hkv=1, D=4, dtype="fp32")
    # 17 tokens need two 16-token blocks; the second holds one row
    assert (n + BLOCK_SIZE - 1) // BLOCK_SIZE == 2 == b.MB
    assert n - BLOCK_SIZE == 1


def test_cu_seqlens_cases():
    for case in ("decode", "prefill_no_cache", "extend"):
        g = GOLD["cu_seqlens_q_cases"][case]
        b = make_batch(0, g["q_lens"], g["k_lens"], Hq=2, Hkv=1, D=4, dtype="fp32")
        assert b.cu_seqlens_q.tolist() == g["cu_seqlens_q"]
        if "cu_seqlens_k" in g:
            assert b.cu_seqlens_k.tolist() == g["cu_seqlens_k"]
        if case == "decode":
            assert b.T == b.B      # the shape test the library uses to pick the decode path
        if case == "prefill_no_cache":
            assert np.array_equal(b.cu_seqlens_q, b.cu_seqlens_k)


def test_token_table_to_pages():
    g = GOLD["token_table_to_pages"]
    slots = np.array(g["token_slots"])
    pages = slots[:g["max_seqlen_k"]:g["page_size"]] // g["page_size"]
    assert pages.tolist() == g["pages"]


def test_workload_slots_follow_the_table():
    b = tiny_varlen_fp32()
    for s in range(b.B):
        sl = b.slots[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
        pos = np.arange(int(b.k_lens[s]))
        assert np.array_equal(sl // 16, b.block_table[s, pos // 16])
        assert np.array_equal(sl % 16, pos % 16)
    # every owned block is used exactly once, the poison block by nobody
    used = np.concatenate([b.block_table[s, :(b.k_lens[s] + 15) // 16] for s in range(b.B)])
    assert np.unique(used).size == used.size and b.poison_block not in used


def test_gqa_group_and_named_shapes():
    g = GOLD["gqa"]
    assert g["q_heads"] // g["kv_heads"] == g["group_size"]
    m = GOLD["decode_manifest"]
    assert m["batch_sequences"] == m["batch_tokens"]
    assert m["page_size"] == BLOCK_SIZE
