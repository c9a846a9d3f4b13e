"""kv_store_rope_paged (RoPE + KV store in one pass) against the CPU oracle.

fp32: rotated values within 1e-5 max-abs of the float64 oracle (angles are
formed in double, the rotation in fp32: about 1e-7 relative).  bf16: within
one bf16 unit in the last place of the exact value plus 1e-6 (the kernel
rounds its fp32 result once, to nearest even), and at least 99% of them
bit-equal to the exact value rounded to nearest even.  V rows and the untouched slots are bit-exact.
The attention over rotated keys then meets the usual attention tolerances.
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


STYLES = {"neox": 0, "interleaved": 1}


def _bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy().view(np.uint32)


def _close(got, exact, dtype, what):
    """got: float64 array from the device; exact: float64 oracle values."""
    if dtype == "fp32":
        err = np.max(np.abs(got - exact))
        print(f"[{what}] max|err|={err:.3e}", flush=True)
        assert err <= 1e-5, f"{what}: {err}"
        return
    from workloads import round_to_bf16
    # one bf16 ulp of the exact value, plus the fp32 rotation's own rounding
    # (a few 1e-8 on N(0, 1) inputs; it matters only where x1 cos - x2 sin cancels)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    assert np.all(np.abs(got - exact) <= ulp + 1e-6), f"{what}: off by more than one bf16 ulp"
    same = np.mean(got == round_to_bf16(exact.astype(np.float32)).astype(np.float64))
    print(f"[{what}] bf16 equal to RNE(exact): {same:.5f}", flush=True)
    assert same >= 0.99


def _case(seed, T, Hq, Hkv, D, dtype, NB=None, neg_every=5, pos_hi=200000):
    rng = np.random.default_rng(seed)
    from workloads import round_to_bf16
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    pos = rng.integers(0, pos_hi, size=T).astype(np.int32)
    pos[:min(T, 6)] = [0, 1, 15, 16, 17, 2**31 - 1][:min(T, 6)]   # position edges, the largest int32
    NB = NB or (T + 15) // 16 + 2
    slots = rng.permutation(NB * 16)[:T].astype(np.int32)
    if neg_every:
        slots[::neg_every] = -1
    return q, k, v, pos, slots, NB


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D,rd", [(64, 64), (128, 128), (128, 64), (128, 32), (96, 96), (256, 256), (64, 16)])
@pytest.mark.parametrize("style", ["neox", "interleaved"])
@pytest.mark.parametrize("scale", [1.0, 4.0])
def test_rope_store_matches_oracle(dtype, D, rd, style, scale):
    import attention_kv_store_amd as kvs
    from oracle import kv_store_rope_oracle
    T, Hq, Hkv = 37, 8, 2
    q, k, v, pos, slots, NB = _case(1000 + D + rd + 7 * STYLES[style], T, Hq, Hkv, D, dtype)
    base = 10000.0 if rd != 16 else 500000.0
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qd = torch.from_numpy(q).to(dt).cuda()
    kc = torch.full((NB, 16, Hkv, D), float("nan"), dtype=dt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kvs.kv_store_rope_paged(qd, torch.from_numpy(k).to(dt).cuda(), torch.from_numpy(v).to(dt).cuda(),
                            torch.from_numpy(pos).cuda(), torch.from_numpy(slots).cuda(), kc, vc,
                            rotary_dim=rd, base=base, style=style, pos_scale=scale)
    torch.cuda.synchronize()
    nan_pool = np.full((NB, 16, Hkv, D), np.nan)
    qr, kr_pool, vr_pool = kv_store_rope_oracle(q, k, v, pos, slots, nan_pool, nan_pool, rotary_dim=rd, base=base,
                                                style=STYLES[style], pos_scale=scale)
    _close(qd.double().cpu().numpy(), qr, dtype, f"q {dtype} D{D} rd{rd} {style} x{scale}")
    live = slots >= 0
    s = slots[live]
    kc_h = kc.double().cpu().numpy().reshape(NB * 16, Hkv, D)
    _close(kc_h[s], kr_pool.reshape(NB * 16, Hkv, D)[s], dtype, "stored k")
    # V is a copy: bit for bit
    vb = _bits(vc).reshape(NB * 16, Hkv, D)
    vsrc = _bits(torch.from_numpy(v).to(dt))
    assert np.array_equal(vb[s], vsrc[live])
    # dims past rotary_dim of K are copies too
    kb = _bits(kc).reshape(NB * 16, Hkv, D)
    ksrc = _bits(torch.from_numpy(k).to(dt))
    assert np.array_equal(kb[s][..., rd:], ksrc[live][..., rd:])
    # every other slot untouched
    other = np.setdiff1d(np.arange(NB * 16), s)
    assert np.isnan(kc.float().cpu().numpy().reshape(NB * 16, -1)[other]).all()
    assert np.isnan(vc.float().cpu().numpy().reshape(NB * 16, -1)[other]).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_rope_without_query_and_without_slots(dtype):
    """q = None rotates and stores K only; all-negative slots rotate q only."""
    import attention_kv_store_amd as kvs
    from oracle import apply_rope
    T, Hq, Hkv, D = 20, 4, 2, 128
    q, k, v, pos, slots, NB = _case(1100, T, Hq, Hkv, D, dtype, neg_every=0)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.full((NB, 16, Hkv, D), float("nan"), dtype=dt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kd, vd = torch.from_numpy(k).to(dt).cuda(), torch.from_numpy(v).to(dt).cuda()
    kvs.kv_store_rope_paged(None, kd, vd, torch.from_numpy(pos).cuda(), torch.from_numpy(slots).cuda(), kc, vc)
    qd = torch.from_numpy(q).to(dt).cuda()
    none = torch.full((T,), -1, dtype=torch.int32, device="cuda")
    kc2 = torch.full_like(kc, float("nan"))
    kvs.kv_store_rope_paged(qd, kd, vd, torch.from_numpy(pos).cuda(), none, kc2, kc2)
    torch.cuda.synchronize()
    kr = apply_rope(k, pos, rotary_dim=D, base=10000.0)
    _close(kc.double().cpu().numpy().reshape(NB * 16, Hkv, D)[slots], kr, dtype, "k only")
    _close(qd.double().cpu().numpy(), apply_rope(q, pos, rotary_dim=D, base=10000.0), dtype, "q only")
    assert np.isnan(kc2.float().cpu().numpy()).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("style", ["neox", "interleaved"])
def test_rope_then_attention(dtype, style):
    """RoPE + store of every token (the cached prefixes first, then the new rows
    with their queries) followed by attention equals the oracle's attention
    over the oracle's rotated (and storage-rounded) Q and K."""
    import dataclasses

    import attention_kv_store_amd as kvs
    from oracle import apply_rope
    from tests.gpu_side import to_f64
    from tests.oracle_side import oracle_attention
    from tests.test_gpu_parity import TOL
    from workloads import make_batch, round_to_bf16
    b = make_batch(1200, [17, 64, 1, 100], [17, 200, 33, 300], Hq=8, Hkv=2, D=128, dtype=dtype, causal=True)
    kw = dict(rotary_dim=128, base=10000.0, style=STYLES[style])
    # positions: a token's key index within its sequence
    kpos = np.concatenate([np.arange(int(n)) for n in b.k_lens]).astype(np.int32)
    qpos = np.concatenate([np.arange(int(lk - lq), int(lk)) for lq, lk in zip(b.q_lens, b.k_lens)]).astype(np.int32)
    rnd = (lambda x: round_to_bf16(x.astype(np.float32)).astype(np.float64)) if dtype == "bf16" else (lambda x: x)
    rb = dataclasses.replace(b, q=rnd(apply_rope(b.q, qpos, **kw)), k_tokens=rnd(apply_rope(b.k_tokens, kpos, **kw)))
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.full(b.pool_shape(), float("nan"), dtype=dt, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    cached, new = b.cached_token_rows(), b.new_token_rows()
    q = torch.from_numpy(b.q).to(dt).cuda()
    put = lambda rows: (torch.from_numpy(b.k_tokens[rows]).to(dt).cuda(), torch.from_numpy(b.v_tokens[rows]).to(dt).cuda(),
                        torch.from_numpy(kpos[rows]).cuda(), torch.from_numpy(b.slots[rows]).cuda())
    if cached.size:
        kn, vn, ps, sl = put(cached)
        kvs.kv_store_rope_paged(None, kn, vn, ps, sl, kc, vc, style=style)
    kn, vn, ps, sl = put(new)
    assert np.array_equal(kpos[new], qpos)
    kvs.kv_store_rope_paged(q, kn, vn, ps, sl, kc, vc, style=style)
    out, lse = kvs.attn_varlen_paged(q, kc, vc, torch.from_numpy(b.block_table).cuda(),
                                     torch.from_numpy(b.cu_seqlens_q).cuda(), torch.from_numpy(b.k_lens).cuda(),
                                     b.scale, True)
    torch.cuda.synchronize()
    ro, rl = oracle_attention(rb)
    eo, el = np.max(np.abs(to_f64(out) - ro)), np.max(np.abs(to_f64(lse) - rl))
    print(f"[rope+attention {dtype} {style}] max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL[dtype] and el <= TOL[dtype]


# ------------------------------------------- RoPE inside the fused decode step --
@pytest.mark.parametrize("D,rd,style", [(64, 64, "neox"), (128, 128, "neox"), (128, 64, "neox"),
                                        (64, 16, "interleaved"), (128, 128, "interleaved")])
@pytest.mark.parametrize("heads", [(8, 2), (32, 8)])
@pytest.mark.parametrize("window,splits", [(0, 0), (0, 7), (33, 0)])
def test_fused_decode_rope(D, rd, style, heads, window, splits):
    """attn_decode_append_paged with rope: out / lse against the oracle's
    attention over the rotated (bf16-rounded) query and new key at position
    Lk - 1; the new key slots hold the rotated key (within a bf16 ulp of the
    exact rotation), the new value slots the value bit for bit, every other
    slot unchanged."""
    import dataclasses

    from oracle import apply_rope
    from tests.gpu_side import cache_bits, run_append, to_device_before_append, to_f64
    from tests.oracle_side import oracle_attention
    from workloads import make_batch, round_to_bf16
    Hq, Hkv = heads
    k_lens = [1, 2, 15, 16, 17, 33, 100, 500, 2000, 64, 65, 31]
    b = make_batch(1700 + D + rd + Hq + window + splits, [1] * len(k_lens), k_lens, Hq=Hq, Hkv=Hkv, D=D,
                   dtype="bf16", causal=True, window=window, name=f"fused-rope-{D}-{rd}-{style}")
    kw = dict(rotary_dim=rd, base=10000.0, style=STYLES[style])
    pos = (b.k_lens - 1).astype(np.int32)
    new = b.new_token_rows()
    rnd = lambda x: round_to_bf16(x.astype(np.float32)).astype(np.float64)
    k_tok = b.k_tokens.astype(np.float64).copy()
    k_exact = apply_rope(b.k_tokens[new], pos, **kw)
    k_tok[new] = rnd(k_exact)
    rb = dataclasses.replace(b, q=rnd(apply_rope(b.q, pos, **kw)), k_tokens=k_tok)
    db, kn, vn = to_device_before_append(b)
    before = cache_bits(db.k_cache).copy()
    q_before = db.q.clone()
    out, lse = run_append(db, kn, vn, window=window, num_splits=splits,
                          rope=dict(rotary_dim=rd, style=style, base=10000.0))
    assert torch.equal(db.q, q_before), "q must not be modified"
    ro, rl = oracle_attention(rb)
    eo, el = np.max(np.abs(to_f64(out) - ro)), np.max(np.abs(to_f64(lse) - rl))
    print(f"[fused rope {D}/{rd}/{style} {Hq}/{Hkv} w{window} s{splits}] max|dout|={eo:.3e} max|dlse|={el:.3e}",
          flush=True)
    assert eo <= 2e-2 and el <= 2e-2
    # the cache: new K rows rotated, new V rows as given, nothing else touched
    slots = b.slots[new]
    kc = to_f64(db.k_cache).reshape(b.num_blocks * 16, Hkv, D)
    _close(kc[slots], k_exact, "bf16", "new key rows")
    vbits = cache_bits(db.v_cache).reshape(b.num_blocks * 16, Hkv, D)
    assert np.array_equal(vbits[slots], _bits(torch.from_numpy(b.v_tokens[new]).to(torch.bfloat16)))
    after = cache_bits(db.k_cache).reshape(b.num_blocks * 16, -1)
    other = np.setdiff1d(np.arange(b.num_blocks * 16), slots)
    assert np.array_equal(after[other], before.reshape(b.num_blocks * 16, -1)[other])
