// Drives every entry point of include/kvstore.h through valid and invalid
// descriptors (fake, never dereferenced device pointers) in a host-only build
// of the C-ABI code under AddressSanitizer / UndefinedBehaviorSanitizer
// (stubs.cpp stands in for the kernels and the HIP runtime).  Exits non-zero
// if a call returns an unexpected status; the sanitizers abort on any memory
// error or undefined behaviour they see.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <vector>

#include "kvstore.h"

static int g_fail = 0;
static kvs_stream_t S = nullptr;

static kvs_tensor T(std::initializer_list<int64_t> shape, int dtype, uintptr_t data = 0x100000) {
  kvs_tensor t;
  std::memset(&t, 0, sizeof t);
  t.data = reinterpret_cast<void*>(data);
  t.dtype = dtype;
  t.ndim = (int32_t)shape.size();
  int i = 0;
  for (int64_t s : shape) t.shape[i++] = s;
  int64_t acc = 1;
  for (int d = t.ndim - 1; d >= 0; --d) {
    t.stride[d] = acc;
    acc *= t.shape[d];
  }
  return t;
}

static void expect(const char* what, kvs_status got, kvs_status want) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, kvs_last_error());
    ++g_fail;
  }
  (void)kvs_last_dispatch();
}

struct Attn {
  kvs_tensor q, k, v, table, cu, lk, out, lse;
};
static Attn attn(int64_t T_, int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int dt, int cache_dt = -1) {
  const int cd = cache_dt < 0 ? dt : cache_dt;
  return {T({T_, Hq, D}, dt), T({64, 16, Hkv, D}, cd), T({64, 16, Hkv, D}, cd), T({B, 8}, KVS_I32),
          T({B + 1}, KVS_I32), T({B}, KVS_I32), T({T_, Hq, D}, dt), T({T_, Hq}, KVS_F32)};
}

static kvs_status call_plain(Attn& a, bool lse = true) {
  return attn_varlen_paged(&a.q, &a.k, &a.v, &a.table, &a.cu, &a.lk, 0.125f, 1, &a.out, lse ? &a.lse : nullptr, S);
}
static kvs_status call_ex(Attn& a, const kvs_hints* h, std::vector<unsigned char>& ws, int window = 0) {
  void* p = ws.empty() ? nullptr : ws.data();
  if (window)
    return attn_varlen_paged_window_ex(&a.q, &a.k, &a.v, &a.table, &a.cu, &a.lk, 0.125f, window, &a.out, &a.lse, h, p,
                                       ws.size(), S);
  return attn_varlen_paged_ex(&a.q, &a.k, &a.v, &a.table, &a.cu, &a.lk, 0.125f, 1, &a.out, &a.lse, h, p, ws.size(), S);
}
static std::vector<unsigned char> workspace(Attn& a, const kvs_hints* h) {
  const size_t n = attn_varlen_paged_workspace_size(&a.q, &a.k, &a.table, h);
  if (n == (size_t)-1) {
    std::fprintf(stderr, "FAIL workspace size refused valid shapes (%s)\n", kvs_last_error());
    ++g_fail;
    return {};
  }
  // host memory stands in for device memory: only its address and size matter
  std::vector<unsigned char> ws(n + 256);
  return ws;
}

int main() {
  // ---- store calls
  for (int dt : {KVS_BF16, KVS_F32}) {
    kvs_tensor kn = T({5, 2, 64}, dt), vn = T({5, 2, 64}, dt), sl = T({5}, KVS_I32);
    kvs_tensor kc = T({8, 16, 2, 64}, dt), vc = T({8, 16, 2, 64}, dt);
    expect("store", kv_store_paged(&kn, &vn, &sl, &kc, &vc, S), KVS_OK);
    kvs_tensor e = T({0, 2, 64}, dt), es = T({0}, KVS_I32);
    expect("store empty", kv_store_paged(&e, &e, &es, &kc, &vc, S), KVS_OK);
    expect("store null", kv_store_paged(nullptr, &vn, &sl, &kc, &vc, S), KVS_ERR_INVALID);
    kvs_tensor bad = kc;
    bad.shape[1] = 32;
    bad.stride[0] = 32 * 2 * 64;
    expect("store page", kv_store_paged(&kn, &vn, &sl, &bad, &bad, S), KVS_ERR_UNSUPPORTED);
    kvs_tensor mis = kn;
    mis.data = reinterpret_cast<void*>(0x100004);
    expect("store align", kv_store_paged(&mis, &vn, &sl, &kc, &vc, S), KVS_ERR_INVALID);
    kvs_rope rope{0, KVS_ROPE_NEOX, 10000.0, 1.0};
    kvs_tensor q = T({5, 8, 64}, dt), pos = T({5}, KVS_I32);
    expect("rope store", kv_store_rope_paged(&q, &kn, &vn, &pos, &sl, &kc, &vc, &rope, S), KVS_OK);
    rope.rotary_dim = 24;
    expect("rope bad dim", kv_store_rope_paged(&q, &kn, &vn, &pos, &sl, &kc, &vc, &rope, S), KVS_ERR_INVALID);
    expect("rope null", kv_store_rope_paged(&q, &kn, &vn, &pos, &sl, &kc, &vc, nullptr, S), KVS_ERR_INVALID);
  }
  for (int code : {KVS_FP8_E4M3, KVS_INT8}) {
    kvs_tensor kn = T({5, 2, 128}, KVS_BF16), vn = T({5, 2, 128}, KVS_BF16), sl = T({5}, KVS_I32);
    kvs_tensor kc = T({8, 16, 2, 128}, code), vc = T({8, 16, 2, 128}, code);
    kvs_tensor ks = T({8, 2, 16}, KVS_F32), vs = T({8, 2, 16}, KVS_F32);
    auto st = code == KVS_INT8 ? kv_store_paged_int8 : kv_store_paged_fp8;
    expect("q8 store", st(&kn, &vn, &sl, &kc, &vc, &ks, &vs, S), KVS_OK);
    kvs_tensor badscale = T({8, 2, 8}, KVS_F32);
    expect("q8 store scales", st(&kn, &vn, &sl, &kc, &vc, &badscale, &vs, S), KVS_ERR_INVALID);
  }

  // ---- attention: prefill / extend and decode paths, both dtypes and head dims
  for (int dt : {KVS_BF16, KVS_F32})
    for (int64_t D : {64, 128}) {
      Attn p = attn(40, 3, 8, 2, D, dt);
      expect("prefill plain", call_plain(p), KVS_OK);
      expect("prefill plain no lse", call_plain(p, false), KVS_OK);
      std::vector<unsigned char> none;
      expect("prefill ex", call_ex(p, nullptr, none), KVS_OK);
      expect("prefill window", call_ex(p, nullptr, none, 33), KVS_OK);
      Attn d = attn(6, 6, 32, 8, D, dt);
      expect("decode plain", call_plain(d), KVS_OK);
      expect("decode noalloc", attn_varlen_paged_noalloc(&d.q, &d.k, &d.v, &d.table, &d.cu, &d.lk, 0.125f, 1, &d.out,
                                                          &d.lse, S),
             KVS_OK);
      expect("prefill noalloc", attn_varlen_paged_noalloc(&p.q, &p.k, &p.v, &p.table, &p.cu, &p.lk, 0.125f, 1,
                                                           &p.out, nullptr, S),
             KVS_OK);
      Attn huge = attn(4096, 4096, 32, 8, D, dt);
      expect("noalloc beyond its scratch", attn_varlen_paged_noalloc(&huge.q, &huge.k, &huge.v, &huge.table, &huge.cu,
                                                                     &huge.lk, 0.125f, 1, &huge.out, &huge.lse, S),
             KVS_ERR_WORKSPACE);
      kvs_hints h{0, 0, 64, 0};
      auto ws = workspace(d, &h);
      expect("decode ex", call_ex(d, &h, ws), KVS_OK);
      std::vector<unsigned char> small(64);
      expect("decode ex small workspace", call_ex(d, &h, small), KVS_ERR_WORKSPACE);
      // mixed batch with its decode rows declared
      Attn m = attn(43, 6, 8, 2, D, dt);
      kvs_hints t{0, 0, 7, 3};
      auto wm = workspace(m, &t);
      expect("decode_tail", call_ex(m, &t, wm), KVS_OK);
      kvs_hints big{0, 0, 0, 9};
      expect("decode_tail too large", call_ex(m, &big, wm), KVS_ERR_INVALID);
      kvs_tensor kn = T({6, 8, D}, dt), vn = T({6, 8, D}, dt);
      expect("append", attn_decode_append_paged(&d.q, &kn, &vn, &d.k, &d.v, &d.table, &d.lk, 0.125f, &d.out, &d.lse,
                                                &h, ws.data(), ws.size(), S),
             KVS_OK);
      expect("append window", attn_decode_append_paged_window(&d.q, &kn, &vn, &d.k, &d.v, &d.table, &d.lk, 0.125f, 5,
                                                               &d.out, &d.lse, &h, ws.data(), ws.size(), S),
             KVS_OK);
      kvs_rope rope{0, KVS_ROPE_NEOX, 10000.0, 1.0};
      expect("append rope", attn_decode_append_paged_rope(&d.q, &kn, &vn, &d.k, &d.v, &d.table, &d.lk, 0.125f, 0,
                                                           &rope, &d.out, &d.lse, &h, ws.data(), ws.size(), S),
             dt == KVS_BF16 ? KVS_OK : KVS_ERR_UNSUPPORTED);
    }
  // quantized caches
  for (int code : {KVS_FP8_E4M3, KVS_INT8}) {
    Attn p = attn(40, 3, 8, 2, 128, KVS_BF16, code);
    kvs_tensor ks = T({64, 2, 16}, KVS_F32), vs = T({64, 2, 16}, KVS_F32);
    auto fn = code == KVS_INT8 ? attn_varlen_paged_int8_ex : attn_varlen_paged_fp8_ex;
    expect("q8 prefill", fn(&p.q, &p.k, &p.v, &ks, &vs, &p.table, &p.cu, &p.lk, 0.1f, 1, 0, &p.out, &p.lse, nullptr,
                            nullptr, 0, S),
           KVS_OK);
    Attn d = attn(5, 5, 8, 2, 128, KVS_BF16, code);
    kvs_hints h{0, 0, 16, 0};
    auto ws = workspace(d, &h);
    expect("q8 decode", fn(&d.q, &d.k, &d.v, &ks, &vs, &d.table, &d.cu, &d.lk, 0.1f, 1, 7, &d.out, &d.lse, &h,
                           ws.data(), ws.size(), S),
           KVS_OK);
    kvs_tensor kn = T({5, 2, 128}, KVS_BF16), vn = T({5, 2, 128}, KVS_BF16);
    auto fused = code == KVS_INT8 ? attn_decode_append_paged_int8 : attn_decode_append_paged_fp8;
    expect("q8 append", fused(&d.q, &kn, &vn, &d.k, &d.v, &ks, &vs, &d.table, &d.lk, 0.1f, 0, &d.out, &d.lse, &h,
                              ws.data(), ws.size(), S),
           KVS_OK);
    Attn plain = attn(5, 5, 8, 2, 128, KVS_BF16, code);
    expect("q8 through the bf16 call", call_plain(plain), KVS_ERR_INVALID);
  }

  // ---- malformed descriptors and arguments
  {
    Attn a = attn(40, 3, 8, 2, 64, KVS_BF16);
    Attn b = a;
    b.q.dtype = 99;
    expect("bad dtype", call_plain(b), KVS_ERR_INVALID);
    b = a;
    b.q.dtype = -1;
    expect("negative dtype", call_plain(b), KVS_ERR_INVALID);
    b = a;
    b.q.ndim = 7;
    expect("bad rank", call_plain(b), KVS_ERR_INVALID);
    b = a;
    b.k.shape[2] = 3;
    b.v.shape[2] = 3;
    expect("Hq % Hkv", call_plain(b), KVS_ERR_INVALID);
    b = a;
    b.q.shape[0] = -5;
    expect("negative extent", call_plain(b), KVS_ERR_INVALID);
    b = a;
    b.q.stride[0] = 7;
    expect("not dense", call_plain(b), KVS_ERR_INVALID);
    b = a;
    b.out.data = nullptr;
    expect("null data", call_plain(b), KVS_ERR_INVALID);
    b = a;
    b.q.shape[0] = INT64_MAX / 2;
    b.q.stride[1] = 0;
    expect("huge extent", call_plain(b), KVS_ERR_INVALID);
    b = a;
    b.table.shape[1] = INT64_MAX / 4;
    b.table.stride[0] = INT64_MAX / 4;
    expect("impossible table", call_plain(b), KVS_ERR_INVALID);
    b = a;
    b.table.shape[1] = int64_t(1) << 31;
    b.table.stride[0] = int64_t(1) << 31;
    expect("table past 32-bit indices", call_plain(b), KVS_ERR_UNSUPPORTED);
    b = a;
    b.q.shape[2] = 96;
    b.q.stride[1] = 96;
    b.q.stride[0] = 8 * 96;
    expect("head dim mismatch", call_plain(b), KVS_ERR_INVALID);
    expect("null q", attn_varlen_paged(nullptr, &a.k, &a.v, &a.table, &a.cu, &a.lk, 0.1f, 1, &a.out, &a.lse, S),
           KVS_ERR_INVALID);
    std::vector<unsigned char> none;
    kvs_hints neg{0, 0, -1, 0};
    expect("negative hints", call_ex(a, &neg, none), KVS_ERR_INVALID);
    expect("window 0", call_ex(a, nullptr, none, -3), KVS_ERR_INVALID);
    const kvs_hints negh{-1, 0, 0, 0};
    if (attn_varlen_paged_workspace_size(&a.q, &a.k, &a.table, &negh) != (size_t)-1) {
      std::fprintf(stderr, "FAIL workspace size accepted negative hints\n");
      ++g_fail;
    }
    float nan = 0.f / 0.f;
    expect("nan scale", attn_varlen_paged(&a.q, &a.k, &a.v, &a.table, &a.cu, &a.lk, nan, 1, &a.out, &a.lse, S),
           KVS_ERR_INVALID);
  }
  expect("release", kvs_release_workspace(), KVS_OK);
  expect("release twice", kvs_release_workspace(), KVS_OK);
  if (g_fail) {
    std::fprintf(stderr, "%d unexpected statuses\n", g_fail);
    return 1;
  }
  std::printf("abi sanitize driver: OK\n");
  return 0;
}
