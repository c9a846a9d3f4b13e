"""FP8 (E4M3) KV cache on the HIP path against the CPU oracle.

The quantizing store is bit-exact: codes and fp32 scales equal the oracle's
(both take x / s and absmax / 448 in fp32).  Attention over the FP8 cache is
compared with the oracle's attention over the dequantized pool
(E4M3(code) * scale) at the bf16 tolerance (max-abs 2e-2 on out and lse).
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
    kc = torch.full((NB, 16, Hkv, D), 0x7F, dtype=torch.uint8, device="cuda")     # NaN codes
    ks = torch.full((NB, Hkv, 16), float("nan"), dtype=torch.float32, device="cuda")
    return kc, kc.clone(), ks, ks.clone()


def _host_pool(NB, Hkv, D):
    kc = np.full((NB, 16, Hkv, D), 0x7F, np.uint8)
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
    k[1, 0, 5] = 300.0                               # one large value: the rest falls in the subnormal range
    v[2, -1, :7] = [0.5, -0.5, 1.5, 2.5, -3.5, 0.25, 448.0]   # values on and between grid points
    if dtype == "bf16":
        k, v = round_to_bf16(k), round_to_bf16(v)
    return k, v


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_store_bitwise(dtype, D):
    import attention_kv_store_amd as kvs
    from oracle import kv_store_fp8_oracle
    T, Hkv, NB = 45, 4, 5
    k, v = _rows(1300 + D, T, Hkv, D, dtype)
    slots = np.random.default_rng(7).permutation(NB * 16)[:T].astype(np.int32)
    slots[3::7] = -1
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = _dev_pool(NB, Hkv, D)
    kvs.kv_store_paged_fp8(torch.from_numpy(k).to(dt).cuda(), torch.from_numpy(v).to(dt).cuda(),
                           torch.from_numpy(slots).cuda(), *dev)
    torch.cuda.synchronize()
    host = kv_store_fp8_oracle(k, v, slots, *_host_pool(NB, Hkv, D))
    _same_pools(dev, host)


def _fp8_batch_pools(b):
    """The batch's every key row stored through kv_store_paged_fp8; returns the
    device pools and the oracle's (after checking they are the same bits)."""
    import attention_kv_store_amd as kvs
    from oracle import kv_store_fp8_oracle
    rows = b.store_rows()
    dev = _dev_pool(b.num_blocks, b.Hkv, b.D)
    kvs.kv_store_paged_fp8(torch.from_numpy(b.k_tokens[rows]).to(torch.bfloat16).cuda(),
                           torch.from_numpy(b.v_tokens[rows]).to(torch.bfloat16).cuda(),
                           torch.from_numpy(b.slots[rows]).cuda(), *dev)
    torch.cuda.synchronize()
    host = kv_store_fp8_oracle(b.k_tokens[rows], b.v_tokens[rows], b.slots[rows], *_host_pool(b.num_blocks, b.Hkv, b.D))
    _same_pools(dev, host)
    return dev, host


def _check_fp8_attention(b, dev, host, rows=None, causal=True, **kw):
    import attention_kv_store_amd as kvs
    from oracle import attention_oracle, dequantize_pool
    from tests.gpu_side import to_f64
    q = torch.from_numpy(b.q).to(torch.bfloat16).cuda()
    out, lse = kvs.attn_varlen_paged_fp8(q, dev[0], dev[1], dev[2], dev[3], torch.from_numpy(b.block_table).cuda(),
                                         torch.from_numpy(b.cu_seqlens_q).cuda(), torch.from_numpy(b.k_lens).cuda(),
                                         b.scale, causal, window=b.window, **kw)
    torch.cuda.synchronize()
    kq, vq, ks, vs = host
    ro, rl = attention_oracle(b.q, dequantize_pool(kq, ks), dequantize_pool(vq, vs), b.block_table, b.cu_seqlens_q,
                              b.k_lens, b.scale, causal, window=b.window, rows=rows)
    go, gl = to_f64(out), to_f64(lse)
    if rows is not None:
        ro, rl, go, gl = ro[rows], rl[rows], go[rows], gl[rows]
    assert np.isfinite(go).all() and np.isfinite(gl).all()
    eo, el = np.max(np.abs(go - ro)), np.max(np.abs(gl - rl))
    print(f"[fp8 {b.name}] max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL and el <= TOL


DECODE_K = [1, 2, 15, 16, 17, 33, 100, 500, 2000, 64, 65, 31]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", [(8, 2), (32, 8), (4, 4)])
@pytest.mark.parametrize("splits", [0, 1, 7, 64])
def test_fp8_decode(D, heads, splits):
    from workloads import make_batch
    Hq, Hkv = heads
    b = make_batch(1400 + D + Hq + splits, [1] * len(DECODE_K), DECODE_K, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                   name=f"decode-D{D}-{Hq}/{Hkv}-s{splits}")
    dev, host = _fp8_batch_pools(b)
    _check_fp8_attention(b, dev, host, num_splits=splits)


@pytest.mark.parametrize("W", [1, 17, 100])
def test_fp8_decode_window(W):
    from workloads import make_batch
    b = make_batch(1450 + W, [1] * len(DECODE_K), DECODE_K, Hq=8, Hkv=2, D=128, dtype="bf16", window=W,
                   name=f"decode-window{W}")
    dev, host = _fp8_batch_pools(b)
    for splits in (0, 7):
        _check_fp8_attention(b, dev, host, num_splits=splits)


def test_fp8_decode_named_workload():
    """The 64-sequence decode workload (contexts 128..2048, 32 / 8 heads, D 64)
    over an FP8 cache."""
    from workloads import paged_decode_bf16
    b = paged_decode_bf16()
    dev, host = _fp8_batch_pools(b)
    _check_fp8_attention(b, dev, host)


PREFILL_Q = [1, 17, 64, 65, 100, 200, 30, 129]
PREFILL_K = [1, 17, 64, 65, 300, 200, 500, 129]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", [(8, 2), (32, 8), (4, 4), (12, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_prefill(D, heads, causal):
    """Prefill and extend rows (cached prefixes over several tiles, a one-row
    sequence, ragged tails) over an FP8 cache."""
    from workloads import make_batch
    Hq, Hkv = heads
    b = make_batch(1470 + D + Hq + causal, PREFILL_Q, PREFILL_K, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", causal=causal,
                   name=f"prefill-D{D}-{Hq}/{Hkv}-{'causal' if causal else 'full'}")
    dev, host = _fp8_batch_pools(b)
    _check_fp8_attention(b, dev, host, causal=causal)


@pytest.mark.parametrize("W", [1, 17, 64, 130])
def test_fp8_prefill_window(W):
    from workloads import make_batch
    b = make_batch(1480 + W, PREFILL_Q, PREFILL_K, Hq=8, Hkv=2, D=128, dtype="bf16", window=W,
                   name=f"prefill-window{W}")
    dev, host = _fp8_batch_pools(b)
    _check_fp8_attention(b, dev, host)


@pytest.mark.parametrize("name", ["causal_prefill_bf16", "mixed_prefill_decode_bf16"])
def test_fp8_named_prefill_workloads(name):
    """The 16 x 512 causal prefill and the mixed 2 x 256 + 30 x 1 batch over an
    FP8 cache, every row."""
    from workloads import NAMED
    b = NAMED[name]()
    dev, host = _fp8_batch_pools(b)
    _check_fp8_attention(b, dev, host)


def test_fp8_decode_tail():
    """An FP8 cache under a mixed batch with its decode rows declared."""
    from workloads import make_batch
    b = make_batch(1490, [40, 17, 1, 1, 1, 1], [40, 100, 1, 17, 700, 2000], Hq=8, Hkv=2, D=128, dtype="bf16",
                   name="fp8-decode-tail")
    dev, host = _fp8_batch_pools(b)
    _check_fp8_attention(b, dev, host, decode_tail=4)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", [(8, 2), (32, 8)])
@pytest.mark.parametrize("window,splits", [(0, 0), (0, 7), (0, 64), (33, 0)])
def test_fp8_fused_decode_step(heads, window, splits, D):
    """attn_decode_append_paged_fp8: the pool afterwards (codes and scales) is
    bit for bit the oracle's quantizing store of every row, the new ones
    included; out / lse match the oracle's attention over it."""
    import attention_kv_store_amd as kvs
    from oracle import kv_store_fp8_oracle
    from workloads import make_batch
    Hq, Hkv = heads
    k_lens = [1, 2, 15, 16, 17, 33, 100, 500, 2000, 64, 65, 31]
    b = make_batch(1750 + Hq + window + splits + D, [1] * len(k_lens), k_lens, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                   window=window, name=f"fp8-fused-{Hq}/{Hkv}-d{D}-w{window}-s{splits}")
    cached = np.intersect1d(b.store_rows(), b.cached_token_rows())
    new = b.new_token_rows()
    dev = _dev_pool(b.num_blocks, b.Hkv, b.D)
    if cached.size:
        kvs.kv_store_paged_fp8(torch.from_numpy(b.k_tokens[cached]).to(torch.bfloat16).cuda(),
                               torch.from_numpy(b.v_tokens[cached]).to(torch.bfloat16).cuda(),
                               torch.from_numpy(b.slots[cached]).cuda(), *dev)
    q = torch.from_numpy(b.q).to(torch.bfloat16).cuda()
    kn = torch.from_numpy(b.k_tokens[new]).to(torch.bfloat16).cuda()
    vn = torch.from_numpy(b.v_tokens[new]).to(torch.bfloat16).cuda()
    out, lse = kvs.attn_decode_append_paged_fp8(q, kn, vn, dev[0], dev[1], dev[2], dev[3],
                                                torch.from_numpy(b.block_table).cuda(),
                                                torch.from_numpy(b.k_lens).cuda(), b.scale, window=window,
                                                num_splits=splits)
    torch.cuda.synchronize()
    rows = b.store_rows()
    host = kv_store_fp8_oracle(b.k_tokens[rows], b.v_tokens[rows], b.slots[rows],
                               *_host_pool(b.num_blocks, b.Hkv, b.D))
    _same_pools(dev, host)
    from oracle import attention_oracle, dequantize_pool
    from tests.gpu_side import to_f64
    ro, rl = attention_oracle(b.q, dequantize_pool(host[0], host[2]), dequantize_pool(host[1], host[3]),
                              b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, True, window=window)
    eo, el = np.max(np.abs(to_f64(out) - ro)), np.max(np.abs(to_f64(lse) - rl))
    print(f"[fp8 fused {Hq}/{Hkv} d{D} w{window} s{splits}] max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL and el <= TOL
