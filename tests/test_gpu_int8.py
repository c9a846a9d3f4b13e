"""INT8 KV cache on the HIP path against the CPU oracle.

The quantizing store is bit-exact: codes and fp32 scales equal the oracle's
(both take x / s and absmax / 127 in fp32, nearest integer ties to even).
Attention over the INT8 cache is compared with the oracle's attention over
the dequantized pool (code * scale) at the bf16 tolerance (max-abs 2e-2 on
out and lse).
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_kv_store_amd._lib as L
    L.load()


TOL = 2e-2


def _dev_pool(NB, Hkv, D):
    kc = torch.full((NB, 16, Hkv, D), -128, dtype=torch.int8, device="cuda")      # a code no store writes
    ks = torch.full((NB, Hkv, 16), float("nan"), dtype=torch.float32, device="cuda")
    return kc, kc.clone(), ks, ks.clone()


def _host_pool(NB, Hkv, D):
    kc = np.full((NB, 16, Hkv, D), -128, np.int8)
    ks = np.full((NB, Hkv, 16), np.nan, np.float32)
    return kc, kc.copy(), ks, ks.copy()


def _same_pools(dev, host):
    for d, h in zip(dev, host):
        d = d.cpu().numpy()
        if d.dtype == np.float32:
            assert np.array_equal(d.view(np.uint32), h.view(np.uint32)), "scales differ"
        else:
            assert np.array_equal(d, h), f"codes differ at {np.argwhere(d != h)[:5].tolist()}"


def _rows(seed, T, Hkv, D, dtype):
    from workloads import round_to_bf16
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((T, Hkv, D)) * np.exp2(rng.uniform(-6, 6, size=(T, Hkv, 1)))).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    k[0, 0] = 0.0                                    # an all-zero row
    k[1, 0] = 1e-3
    k[1, 0, 5] = 300.0                               # one large value: the rest rounds to 0
    v[2, -1, :] = 0.0
    v[2, -1, :8] = [127.0, -0.5, 0.5, 1.5, 2.5, -2.5, 126.5, -127.0]   # s = 1: exact halves, ties to even
    if dtype == "bf16":
        k, v = round_to_bf16(k), round_to_bf16(v)
    return k, v


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
def test_int8_store_bitwise(dtype, D):
    import attention_kv_store_amd as kvs
    from oracle import kv_store_int8_oracle
    T, Hkv, NB = 45, 4, 5
    k, v = _rows(1600 + D, T, Hkv, D, dtype)
    slots = np.random.default_rng(8).permutation(NB * 16)[:T].astype(np.int32)
    slots[3::7] = -1
    slots[2] = 17                                    # the row with the hand-picked halves is stored
    slots[np.arange(T) != 2] = np.where(slots[np.arange(T) != 2] == 17, -1, slots[np.arange(T) != 2])
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = _dev_pool(NB, Hkv, D)
    kvs.kv_store_paged_int8(torch.from_numpy(k).to(dt).cuda(), torch.from_numpy(v).to(dt).cuda(),
                            torch.from_numpy(slots).cuda(), *dev)
    torch.cuda.synchronize()
    host = kv_store_int8_oracle(k, v, slots, *_host_pool(NB, Hkv, D))
    _same_pools(dev, host)
    # the halves of row 2's last head landed on the even integers
    assert host[1][1, 1, -1, :8].tolist() == [127, 0, 0, 2, 2, -2, 126, -127]


def _int8_batch_pools(b):
    """The batch's every key row stored through kv_store_paged_int8; returns the
    device pools and the oracle's (after checking they are the same bits)."""
    import attention_kv_store_amd as kvs
    from oracle import kv_store_int8_oracle
    rows = b.store_rows()
    dev = _dev_pool(b.num_blocks, b.Hkv, b.D)
    kvs.kv_store_paged_int8(torch.from_numpy(b.k_tokens[rows]).to(torch.bfloat16).cuda(),
                            torch.from_numpy(b.v_tokens[rows]).to(torch.bfloat16).cuda(),
                            torch.from_numpy(b.slots[rows]).cuda(), *dev)
    torch.cuda.synchronize()
    host = kv_store_int8_oracle(b.k_tokens[rows], b.v_tokens[rows], b.slots[rows],
                                *_host_pool(b.num_blocks, b.Hkv, b.D))
    _same_pools(dev, host)
    return dev, host


def _check_int8_attention(b, dev, host, rows=None, causal=True, **kw):
    import attention_kv_store_amd as kvs
    from oracle import attention_oracle, dequantize_pool_int8
    from tests.gpu_side import to_f64
    q = torch.from_numpy(b.q).to(torch.bfloat16).cuda()
    out, lse = kvs.attn_varlen_paged_int8(q, dev[0], dev[1], dev[2], dev[3], torch.from_numpy(b.block_table).cuda(),
                                          torch.from_numpy(b.cu_seqlens_q).cuda(), torch.from_numpy(b.k_lens).cuda(),
                                          b.scale, causal, window=b.window, **kw)
    torch.cuda.synchronize()
    kq, vq, ks, vs = host
    ro, rl = attention_oracle(b.q, dequantize_pool_int8(kq, ks), dequantize_pool_int8(vq, vs), b.block_table,
                              b.cu_seqlens_q, b.k_lens, b.scale, causal, window=b.window, rows=rows)
    go, gl = to_f64(out), to_f64(lse)
    if rows is not None:
        ro, rl, go, gl = ro[rows], rl[rows], go[rows], gl[rows]
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    eo, el = np.max(np.abs(go - ro)), np.max(np.abs(gl - rl))
    print(f"[int8 {b.name}] max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL and el <= TOL


DECODE_K = [1, 2, 15, 16, 17, 33, 100, 500, 2000, 64, 65, 31]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", [(8, 2), (32, 8), (4, 4)])
@pytest.mark.parametrize("splits", [0, 7, 64])
def test_int8_decode(D, heads, splits):
    from workloads import make_batch
    Hq, Hkv = heads
    b = make_batch(1700 + D + Hq + splits, [1] * len(DECODE_K), DECODE_K, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                   name=f"int8-decode-D{D}-{Hq}/{Hkv}-s{splits}")
    dev, host = _int8_batch_pools(b)
    _check_int8_attention(b, dev, host, num_splits=splits)


@pytest.mark.parametrize("W", [1, 100])
def test_int8_decode_window(W):
    from workloads import make_batch
    b = make_batch(1750 + W, [1] * len(DECODE_K), DECODE_K, Hq=8, Hkv=2, D=128, dtype="bf16", window=W,
                   name=f"int8-decode-window{W}")
    dev, host = _int8_batch_pools(b)
    for splits in (0, 7):
        _check_int8_attention(b, dev, host, num_splits=splits)


def test_int8_decode_named_workload():
    """The 64-sequence decode workload (contexts 204..2035, 32 / 8 heads, D 64)
    over an INT8 cache."""
    from workloads import paged_decode_bf16
    b = paged_decode_bf16()
    dev, host = _int8_batch_pools(b)
    _check_int8_attention(b, dev, host)


PREFILL_Q = [1, 17, 64, 65, 100, 200, 30, 129]
PREFILL_K = [1, 17, 64, 65, 300, 200, 500, 129]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", [(8, 2), (32, 8), (12, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_int8_prefill(D, heads, causal):
    """Prefill and extend rows (cached prefixes over several tiles, a one-row
    sequence, ragged tails) over an INT8 cache."""
    from workloads import make_batch
    Hq, Hkv = heads
    b = make_batch(1770 + D + Hq + causal, PREFILL_Q, PREFILL_K, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", causal=causal,
                   name=f"int8-prefill-D{D}-{Hq}/{Hkv}-{'causal' if causal else 'full'}")
    dev, host = _int8_batch_pools(b)
    _check_int8_attention(b, dev, host, causal=causal)


@pytest.mark.parametrize("W", [17, 130])
def test_int8_prefill_window(W):
    from workloads import make_batch
    b = make_batch(1790 + W, PREFILL_Q, PREFILL_K, Hq=8, Hkv=2, D=128, dtype="bf16", window=W,
                   name=f"int8-prefill-window{W}")
    dev, host = _int8_batch_pools(b)
    _check_int8_attention(b, dev, host)


@pytest.mark.parametrize("name", ["causal_prefill_bf16", "mixed_prefill_decode_bf16"])
def test_int8_named_prefill_workloads(name):
    """The 16 x 512 causal prefill and the mixed 2 x 256 + 30 x 1 batch over an
    INT8 cache, every row."""
    from workloads import NAMED
    b = NAMED[name]()
    dev, host = _int8_batch_pools(b)
    _check_int8_attention(b, dev, host)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window,splits", [(0, 0), (0, 7), (0, 64), (33, 0)])
def test_int8_fused_decode_step(D, window, splits):
    """attn_decode_append_paged_int8: the pool afterwards (codes and scales) is
    bit for bit the oracle's quantizing store of every row, the new ones
    included; out / lse match the oracle's attention over it."""
    import attention_kv_store_amd as kvs
    from oracle import attention_oracle, dequantize_pool_int8, kv_store_int8_oracle
    from tests.gpu_side import to_f64
    from workloads import make_batch
    k_lens = [1, 2, 15, 16, 17, 33, 100, 500, 2000, 64, 65, 31]
    b = make_batch(1810 + D + window + splits, [1] * len(k_lens), k_lens, Hq=8, Hkv=2, D=D, dtype="bf16",
                   window=window, name=f"int8-fused-d{D}-w{window}-s{splits}")
    cached = np.intersect1d(b.store_rows(), b.cached_token_rows())
    new = b.new_token_rows()
    dev = _dev_pool(b.num_blocks, b.Hkv, b.D)
    if cached.size:
        kvs.kv_store_paged_int8(torch.from_numpy(b.k_tokens[cached]).to(torch.bfloat16).cuda(),
                                torch.from_numpy(b.v_tokens[cached]).to(torch.bfloat16).cuda(),
                                torch.from_numpy(b.slots[cached]).cuda(), *dev)
    q = torch.from_numpy(b.q).to(torch.bfloat16).cuda()
    kn = torch.from_numpy(b.k_tokens[new]).to(torch.bfloat16).cuda()
    vn = torch.from_numpy(b.v_tokens[new]).to(torch.bfloat16).cuda()
    out, lse = kvs.attn_decode_append_paged_int8(q, kn, vn, dev[0], dev[1], dev[2], dev[3],
                                                 torch.from_numpy(b.block_table).cuda(),
                                                 torch.from_numpy(b.k_lens).cuda(), b.scale, window=window,
                                                 num_splits=splits)
    torch.cuda.synchronize()
    rows = b.store_rows()
    host = kv_store_int8_oracle(b.k_tokens[rows], b.v_tokens[rows], b.slots[rows],
                                *_host_pool(b.num_blocks, b.Hkv, b.D))
    _same_pools(dev, host)
    ro, rl = attention_oracle(b.q, dequantize_pool_int8(host[0], host[2]), dequantize_pool_int8(host[1], host[3]),
                              b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, True, window=window)
    eo, el = np.max(np.abs(to_f64(out) - ro)), np.max(np.abs(to_f64(lse) - rl))
    print(f"[int8 fused d{D} w{window} s{splits}] max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL and el <= TOL


def test_int8_and_fp8_calls_reject_each_others_cache():
    """An INT8 pool handed to the FP8 calls (and back) is refused before any
    launch."""
    import attention_kv_store_amd as kvs
    from workloads import make_batch
    b = make_batch(1830, [1, 1], [5, 40], Hq=8, Hkv=2, D=64, dtype="bf16")
    i8 = _dev_pool(b.num_blocks, b.Hkv, b.D)
    f8 = (torch.zeros_like(i8[0], dtype=torch.uint8), torch.zeros_like(i8[1], dtype=torch.uint8), i8[2], i8[3])
    q = torch.from_numpy(b.q).to(torch.bfloat16).cuda()
    meta = [torch.from_numpy(x).cuda() for x in (b.block_table, b.cu_seqlens_q, b.k_lens)]
    kn = torch.zeros(2, 2, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvs.KvsError):
        kvs.attn_varlen_paged_fp8(q, *i8, *meta, b.scale, True)
    with pytest.raises(kvs.KvsError):
        kvs.attn_varlen_paged_int8(q, *f8, *meta, b.scale, True)
    with pytest.raises(kvs.KvsError):
        kvs.kv_store_paged_fp8(kn, kn, torch.zeros(2, dtype=torch.int32, device="cuda"), *i8)
    with pytest.raises(kvs.KvsError, match="INT8 codes"):
        kvs.attn_decode_append_paged_int8(q, kn, kn, *f8, meta[0], meta[2], b.scale)
    with pytest.raises(kvs.KvsError, match="FP8"):
        kvs.attn_decode_append_paged_fp8(q, kn, kn, *i8, meta[0], meta[2], b.scale)
    with pytest.raises(kvs.KvsError, match="quantized caches need their scales"):
        kvs.attn_varlen_paged(q, i8[0], i8[1], *meta, b.scale, True)
