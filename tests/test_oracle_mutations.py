"""Planted mistakes in a copy of the oracle must each be caught by a pin.

The mutated copies are built from the oracle's source text on the CPU and never
leave this test.  The battery below reuses the facts of test_oracle_pins.py
(multi-precision brute force, torch SDPA, closed forms and the one-hot probe).
"""
from __future__ import annotations

import inspect
import math
import types

import numpy as np
import pytest

import oracle.attention as oa
from tests.oracle_side import gather_loop, oracle_pool
from tests.test_oracle_pins import _brute
from workloads import make_batch

MUTATIONS = {
    "gqa map h % Hkv": ("g = h // G", "g = h % Hkv"),
    "causal off by one": ("<= (cached + i)[:, None]", "< (cached + i)[:, None]"),
    "top-left causal": ("<= (cached + i)[:, None]", "<= i[:, None]"),
    "lse drops max": ("lse[rws, h] = m + np.log(l)", "lse[rws, h] = np.log(l)"),
    "no normalisation": ("/ l[:, None]", "/ 1.0"),
    "scale dropped": ("S = scale * (", "S = ("),
    "k/v swapped": ("(P @ Vb[k0:ncols, g, :])", "(P @ Kb[k0:ncols, g, :])"),
    "block row index": ("cache[blocks, t % block_size]", "cache[blocks, t // block_size % block_size]"),
    "page index": ("[t // block_size]", "[t % block_size]"),
    "transposed q/k": ("(q[rws, h, :] @ Kb[k0:ncols, g, :].T)", "(Kb[:rws.size, g, :] @ q[rws, h, :].T).T[:, k0:ncols]"),
    "max not subtracted in lse": ("P = np.exp(S - m[:, None])", "P = np.exp(S)"),
    "window off by one": (">= (cached + i - window + 1)[:, None]", ">= (cached + i - window)[:, None]"),
    "window from top-left": (">= (cached + i - window + 1)[:, None]", ">= (i - window + 1)[:, None]"),
    "window ignored": ("            if window:\n", "            if False:\n"),
    "window start of the last row": ("cached + int(i.min()) - window + 1", "cached + int(i.max()) - window + 1"),
}


def _mutant(src_from, src_to):
    src = inspect.getsource(oa)
    assert src_from in src, src_from
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(src_from, src_to), "oracle_mutant", "exec"), mod.__dict__)
    return mod.attention_oracle


def _battery(attn):
    """Return True if every pin holds for the given attention function."""
    try:
        # brute force, GQA, cached prefix, causal
        b = make_batch(5, [17, 3], [17, 20], Hq=4, Hkv=2, D=4, dtype="fp32", causal=True)
        kc, vc = oracle_pool(b)
        out, lse = attn(b.q, kc, vc, b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, True)
        for s in range(b.B):
            r0, r1 = int(b.cu_seqlens_q[s]), int(b.cu_seqlens_q[s + 1])
            ks = b.k_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
            vs = b.v_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
            bo, bl = _brute(b.q[r0:r1], ks, vs, r1 - r0, int(b.k_lens[s]), b.scale, True, 2, dps=25)
            if not (np.max(np.abs(out[r0:r1] - bo)) <= 1e-12 and np.max(np.abs(lse[r0:r1] - bl)) <= 1e-12):
                return False
        # torch SDPA, wider D (the brute force case above has D = 4)
        import torch
        import torch.nn.functional as F
        b = make_batch(6, [9, 1], [40, 33], Hq=8, Hkv=2, D=16, dtype="fp32", causal=True)
        kc, vc = oracle_pool(b)
        out, _ = attn(b.q, kc, vc, b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, True)
        for s in range(b.B):
            lq, lk = int(b.q_lens[s]), int(b.k_lens[s])
            r0 = int(b.cu_seqlens_q[s])
            K = torch.from_numpy(gather_loop(kc, b.block_table[s], lk)).permute(1, 0, 2)[None]
            V = torch.from_numpy(gather_loop(vc, b.block_table[s], lk)).permute(1, 0, 2)[None]
            Q = torch.from_numpy(b.q[r0:r0 + lq].astype(np.float64)).permute(1, 0, 2)[None]
            mask = torch.arange(lk)[None, :] <= (lk - lq + torch.arange(lq)[:, None])
            ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=b.scale,
                                                 enable_gqa=True)[0].permute(1, 0, 2).numpy()
            if not np.max(np.abs(out[r0:r0 + lq] - ref)) <= 1e-12:
                return False
        # Q = 0 closed form
        b = make_batch(7, [9], [25], Hq=2, Hkv=1, D=4, dtype="fp32", causal=True)
        b.q[:] = 0
        kc, vc = oracle_pool(b)
        out, lse = attn(b.q, kc, vc, b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, True)
        V = b.v_tokens.astype(np.float64)
        for i in range(9):
            n = 16 + i + 1
            if abs(lse[i, 0] - math.log(n)) > 1e-12 or np.max(np.abs(out[i, 0] - V[:n, 0].mean(0))) > 1e-12:
                return False
        # sliding window: brute force over the band, decode and extend rows
        for W in (1, 3, 20):
            b = make_batch(8, [17, 1, 4], [25, 20, 30], Hq=2, Hkv=1, D=4, dtype="fp32", causal=True, window=W)
            kc, vc = oracle_pool(b)
            out, lse = attn(b.q, kc, vc, b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, True, window=W)
            for s in range(b.B):
                r0, r1 = int(b.cu_seqlens_q[s]), int(b.cu_seqlens_q[s + 1])
                ks = b.k_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
                vs = b.v_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
                bo, bl = _brute(b.q[r0:r1], ks, vs, r1 - r0, int(b.k_lens[s]), b.scale, True, 2, dps=25, window=W)
                if not (np.max(np.abs(out[r0:r1] - bo)) <= 1e-12 and np.max(np.abs(lse[r0:r1] - bl)) <= 1e-12):
                    return False
        return True
    except Exception:
        return False


def test_unmutated_oracle_passes_battery():
    assert _battery(oa.attention_oracle)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    attn = _mutant(*MUTATIONS[name])
    assert not _battery(attn), f"planted mistake '{name}' went unnoticed"
