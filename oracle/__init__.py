"""CPU oracle for paged varlen attention and the paged KV store.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in this
package.  The product path (``attention_kv_store_amd``) never does, and it shares
no code, constants or helpers with this package.

Every function here is a plain numpy float64 transcription of what the pages
define, with no tiling, fusion or reordering beyond that definition:

* ``attention_oracle`` -- softmax(scale * Q K^T + mask) V with the full score rows
  materialised, as in the naive schedule of Transformer 추론 커널 (3/10), §10
  (equation for O), gathered through the block table of §14.
* ``kv_store_oracle`` -- the scatter of new K/V rows into their slots
  (Transformer 추론 커널 (3/10), §2 "RoPE + KV cache store" step; slot = block *
  page_size + offset per 장부가 커널 인자로 바뀌는 지점과 CUDA graph, page-table part).
* ``apply_rope`` / ``kv_store_rope_oracle`` -- the rotary position embedding
  of Q and K and the "RoPE + KV cache store" step (Transformer 추론 커널 (3/10),
  §1-§2, §19, §24; formula from RoFormer, section 3.2 -- the pages give none).
* ``e4m3_encode`` / ``e4m3_decode`` / ``quantize_rows`` / ``kv_store_fp8_oracle``
  / ``dequantize_pool`` -- the FP8 (OCP E4M3) KV cache with one scale per
  token row and KV head (Transformer 추론 커널 (3/10), §7, §19, §24 name FP8 KV,
  quantized layouts and scale layouts; the format is the OCP specification's).
* ``int8_encode`` / ``int8_decode`` / ``quantize_rows_int8`` /
  ``kv_store_int8_oracle`` / ``dequantize_pool_int8`` -- the INT8 KV cache
  with the same scale layout (s = absmax / 127, codes rounded to nearest even
  and clamped to +-127; §19 and §24 name INT8 KV next to FP8).
* ``lse_merge`` -- the stable merge of partial results over disjoint key sets
  (Transformer 추론 커널 (3/10), §12 equations for m_new / l_new, and §16).

Pins (tests/test_oracle_*pins.py) tie every function to something other than
itself: closed forms, invariants, a multi-precision brute force and CPU torch
SDPA.  Where the pages are silent, each module's docstring states the reading
it takes.
"""
from .attention import attention_oracle, gather_sequence, lse_merge, BLOCK_SIZE  # noqa: F401
from .store import kv_store_oracle  # noqa: F401
from .rope import INTERLEAVED, NEOX, apply_rope, kv_store_rope_oracle  # noqa: F401
from .fp8 import dequantize_pool, e4m3_decode, e4m3_encode, kv_store_fp8_oracle, quantize_rows  # noqa: F401
from .int8 import dequantize_pool_int8, int8_decode, int8_encode, kv_store_int8_oracle, quantize_rows_int8  # noqa: F401
