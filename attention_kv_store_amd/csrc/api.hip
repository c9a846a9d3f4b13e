// extern "C" entry points of libkvstore.so: host-side validation, dispatch
// planning and launches.  Validation touches no device memory and makes no HIP
// call, so every error path can be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kvstore.h"
#include "kvs_internal.hpp"

namespace {

// The calling thread's last error and dispatch texts: fixed buffers, so no
// call allocates host memory for them either.
constexpr size_t kTextBytes = 512;
thread_local char g_err[kTextBytes];
thread_local char g_dispatch[kTextBytes];

void clear_error() { g_err[0] = 0; }

kvs_status fail(kvs_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, kTextBytes, fmt, ap);
  va_end(ap);
  return st;
}

void set_dispatch(const char* fmt, ...) {
  char buf[kTextBytes];   // the arguments may be g_dispatch itself
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  memcpy(g_dispatch, buf, sizeof buf);
}

const char* dtname(int dt) {
  switch (dt) {
    case KVS_F32: return "f32";
    case KVS_BF16: return "bf16";
    case KVS_I32: return "i32";
    case KVS_FP8_E4M3: return "fp8_e4m3";
    case KVS_INT8: return "int8";
    default: return "?";
  }
}

int esize(int dt) { return dt == KVS_BF16 ? 2 : (dt == KVS_FP8_E4M3 || dt == KVS_INT8 ? 1 : 4); }

// Checks a descriptor: present, dtype in `allowed` (bitmask of 1 << dtype),
// rank, dense row-major strides, alignment.  Returns KVS_OK or sets g_err.
kvs_status check_tensor(const kvs_tensor* t, const char* name, unsigned allowed, int ndim,
                        bool allow_empty = false) {
  if (!t) return fail(KVS_ERR_INVALID, "%s: descriptor is NULL", name);
  if (t->dtype < 0 || t->dtype > KVS_INT8 || !(allowed & (1u << t->dtype)))
    return fail(KVS_ERR_INVALID, "%s: dtype %s not allowed here", name, dtname(t->dtype));
  if (t->ndim != ndim) return fail(KVS_ERR_INVALID, "%s: expected %d dims, got %d", name, ndim, t->ndim);
  // element counts are formed with overflow checks: a descriptor whose
  // extents multiply past 2^62 elements describes no real buffer
  int64_t numel = 1;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return fail(KVS_ERR_INVALID, "%s: negative extent in dim %d", name, i);
    if (__builtin_mul_overflow(numel, t->shape[i], &numel) || numel > (int64_t(1) << 62))
      return fail(KVS_ERR_INVALID, "%s: extents too large", name);
  }
  int64_t expect = 1;
  for (int i = ndim - 1; i >= 0; --i) {
    if (t->shape[i] > 1 && t->stride[i] != expect)
      return fail(KVS_ERR_INVALID, "%s: not dense row-major (dim %d stride %lld, expected %lld)", name, i,
                  (long long)t->stride[i], (long long)expect);
    expect *= t->shape[i];   // bounded by numel above
  }
  if (numel == 0) {
    if (!allow_empty) return fail(KVS_ERR_INVALID, "%s: empty tensor", name);
    return KVS_OK;
  }
  if (!t->data) return fail(KVS_ERR_INVALID, "%s: data pointer is NULL", name);
  const uintptr_t align = t->dtype == KVS_I32 ? 4 : 16;
  if (reinterpret_cast<uintptr_t>(t->data) % align)
    return fail(KVS_ERR_INVALID, "%s: data pointer not %zu-byte aligned", name, (size_t)align);
  return KVS_OK;
}

#define KVS_TRY(expr)                    \
  do {                                   \
    kvs_status _st = (expr);             \
    if (_st != KVS_OK) return _st;       \
  } while (0)

constexpr unsigned kFloatTypes = (1u << KVS_F32) | (1u << KVS_BF16);
constexpr unsigned kCacheTypes = kFloatTypes | (1u << KVS_FP8_E4M3) | (1u << KVS_INT8);   // attention may read FP8 / INT8 caches
constexpr unsigned kIntTypes = (1u << KVS_I32);

// ---- attention plan --------------------------------------------------------
struct Plan {
  kvs::AttnParams p{};
  kvs::DType dt;
  int D = 0;
  bool decode = false;
  // mixed launch (T != B, bf16): prefill items and one-row decode ranges
  // share one grid of mixed_grid workgroups
  bool mixed = false;
  int mixed_grid = 0;
  size_t mixed_lds = 0;
  size_t ws_bytes = 0;   // scratch needed (decode with >1 split, mixed launch)
  size_t ws_po_off = 0;  // byte offset of part_o inside the scratch
  size_t ws_lse_off = 0; // byte offset of part_lse inside the scratch
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- compute units of the current device (cached per device) ---------------
constexpr int kMaxDevices = 64;
std::mutex g_cu_mu;
int g_cus[kMaxDevices];

kvs_status device_cus(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(KVS_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(KVS_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_cu_mu);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      return fail(KVS_ERR_HIP, "hipDeviceGetAttribute(MultiprocessorCount) failed");
    g_cus[dev] = n;
  }
  *out = g_cus[dev];
  return KVS_OK;
}

// Decode LDS budget of one workgroup (160 KiB per CU, less the kernels'
// static LDS).
constexpr size_t kLdsBudget = 160 * 1024 - 256;

// T != B: whether the batch runs as a mixed launch, and its sizes.  bf16
// with KV heads in whole groups of the prefill workgroup's waves (the decode
// part's workgroup is the prefill part's, one wave per KV head); otherwise --
// and when a limit below is exceeded -- the prefill kernel serves every
// sequence, one-row ones included.  A batch of one sequence (then with T > 1
// rows) has no one-row sequence and runs in the prefill kernel too.  The grid
// holds the prefill kernel's workgroups per CU, and at least 8 more than the
// decode ranges a range's table window could need.
kvs_status plan_mixed(Plan* plan, int32_t qdt, bool kv8, int D, int64_t B, int64_t MB) {
  kvs::AttnParams& p = plan->p;
  plan->mixed = false;
  p.mixed = 0;
  const int nw = p.pnw;
  if (qdt != KVS_BF16 || kv8 || (nw != 4 && nw != 8) || p.Hkv % nw || p.G > 16 || B < 2 || B > 8192) return KVS_OK;
  int cus = 0;
  KVS_TRY(device_cus(&cus));
  const int64_t nhg = p.Hkv / nw;
  if (nhg > 64) return KVS_OK;
  const int64_t need = nhg * ((B * MB + kvs::kDecodeTblWin - 1) / kvs::kDecodeTblWin);
  const int64_t W = align_up((size_t)std::max<int64_t>((int64_t)cus * (nw == 4 ? 2 : 1), 8 + need), 8);
  if (W > (1 << 20)) return KVS_OK;
  if (B * p.Hkv > (int64_t)(kvs::kDecodeCounterBytes / sizeof(int32_t))) return KVS_OK;
  if ((double)(W + B) * p.Hq * D * sizeof(float) >= 2147483648.0) return KVS_OK;
  const size_t dec_lds = kvs::decode_lds_bytes((int)B, kvs::decode_tbl_ints((int)B, (int)MB, false) + kvs::decode_mix_ints((int)B),
                                               nw, kvs::decode_slab_bytes(D, false));
  const size_t pre_lds = kvs::prefill_lds_bytes(D, true, (int)B, p.meta_lds);
  if (dec_lds > kLdsBudget || pre_lds > kLdsBudget) return KVS_OK;
  plan->mixed = true;
  plan->mixed_grid = (int)W;
  plan->mixed_lds = std::max(dec_lds, pre_lds);
  p.mixed = 1;
  p.hpw = nw;
  p.nwg = (int32_t)W;   // partial slots: at most W ranges + B sequences
  p.dsmall = 0;
  const size_t slots = (size_t)W + B;
  plan->ws_po_off = kvs::kDecodeCounterBytes;
  plan->ws_lse_off = plan->ws_po_off + align_up(slots * p.Hq * D * sizeof(float), 256);
  plan->ws_bytes = plan->ws_lse_off + align_up(slots * p.Hq * sizeof(float), 256);
  return KVS_OK;
}

// Validates shapes (not device values) and fills the plan.  `v_cache`,
// `cu`, `lk`, `out`, `lse` may be NULL when only sizing the workspace; `cu`
// is NULL in append mode (one query row per sequence).
kvs_status make_plan(const kvs_tensor* q, const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                     const kvs_tensor* table, const kvs_tensor* cu, const kvs_tensor* lk, float scale,
                     int causal, const kvs_tensor* out, const kvs_tensor* lse, const kvs_hints* hints,
                     bool sizing_only, Plan* plan, bool append = false, int window = 0, int64_t rows_bound = 0) {
  KVS_TRY(check_tensor(q, "q", kFloatTypes, 3));
  KVS_TRY(check_tensor(k_cache, "k_cache", kCacheTypes, 4));
  KVS_TRY(check_tensor(table, "block_table", kIntTypes, 2));
  const int64_t T = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  const int64_t NB = k_cache->shape[0], page = k_cache->shape[1], Hkv = k_cache->shape[2];
  const int64_t B = table->shape[0], MB = table->shape[1];
  const bool kv8 = k_cache->dtype == KVS_FP8_E4M3 || k_cache->dtype == KVS_INT8;   // codes: the queries are bf16
  if (kv8 ? q->dtype != KVS_BF16 : k_cache->dtype != q->dtype)
    return fail(KVS_ERR_INVALID, "k_cache dtype %s does not go with q dtype %s", dtname(k_cache->dtype), dtname(q->dtype));
  if (k_cache->shape[3] != D) return fail(KVS_ERR_INVALID, "k_cache head dim %lld != q head dim %lld", (long long)k_cache->shape[3], (long long)D);
  if (page != 16) return fail(KVS_ERR_UNSUPPORTED, "page size %lld not supported (only 16)", (long long)page);
  if (D != 64 && D != 128) return fail(KVS_ERR_UNSUPPORTED, "head dim %lld not supported (64 or 128)", (long long)D);
  if (Hkv < 1 || Hq < 1 || Hq % Hkv) return fail(KVS_ERR_INVALID, "Hq (%lld) must be a positive multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (B < 1) return fail(KVS_ERR_INVALID, "batch must hold at least one sequence");
  if (T < B) return fail(KVS_ERR_INVALID, "total query rows T=%lld < batch B=%lld (every sequence needs >= 1 row)", (long long)T, (long long)B);
  if (MB < 1) return fail(KVS_ERR_INVALID, "block_table needs at least one column");
  if (T > INT32_MAX / 2 || Hq > 4096 || NB * 16 > INT32_MAX || B * MB > INT32_MAX)
    return fail(KVS_ERR_UNSUPPORTED, "sizes beyond the 32-bit index ranges the kernels use");
  if (!sizing_only) {
    KVS_TRY(check_tensor(v_cache, "v_cache", kCacheTypes, 4));
    for (int i = 0; i < 4; ++i)
      if (v_cache->shape[i] != k_cache->shape[i]) return fail(KVS_ERR_INVALID, "v_cache shape != k_cache shape");
    if (v_cache->dtype != k_cache->dtype) return fail(KVS_ERR_INVALID, "v_cache dtype != k_cache dtype");
    if (!append) {
      KVS_TRY(check_tensor(cu, "cu_seqlens_q", kIntTypes, 1));
      if (cu->shape[0] != B + 1) return fail(KVS_ERR_INVALID, "cu_seqlens_q has %lld entries, expected B+1=%lld", (long long)cu->shape[0], (long long)(B + 1));
    } else if (T != B) {
      return fail(KVS_ERR_INVALID, "append mode needs one query row per sequence (q has %lld rows for %lld sequences)", (long long)T, (long long)B);
    }
    KVS_TRY(check_tensor(lk, "seqlens_k", kIntTypes, 1));
    if (lk->shape[0] != B) return fail(KVS_ERR_INVALID, "seqlens_k has %lld entries, expected B=%lld", (long long)lk->shape[0], (long long)B);
    KVS_TRY(check_tensor(out, "out", kFloatTypes, 3));
    if (out->dtype != q->dtype) return fail(KVS_ERR_INVALID, "out dtype != q dtype");
    for (int i = 0; i < 3; ++i)
      if (out->shape[i] != q->shape[i]) return fail(KVS_ERR_INVALID, "out shape != q shape");
    if (lse) {
      KVS_TRY(check_tensor(lse, "lse", 1u << KVS_F32, 2));
      if (lse->shape[0] != T || lse->shape[1] != Hq) return fail(KVS_ERR_INVALID, "lse must be [T, Hq]");
    }
    if (!std::isfinite(scale)) return fail(KVS_ERR_INVALID, "scale must be finite");
  }
  if (window < 0 || (window > 0 && !causal)) return fail(KVS_ERR_INVALID, "window must be >= 1 and needs the causal mask");
  if (window > 0) {
    // every key index is below 16 * MB, so a wider window is the same mask;
    // with both below 2^30 the kernels' window arithmetic stays in 32 bits
    if (16 * MB > (int64_t(1) << 30))
      return fail(KVS_ERR_UNSUPPORTED, "a sliding window needs 16 * MB <= 2^30 (MB = %lld)", (long long)MB);
    window = (int)std::min<int64_t>(window, 16 * MB);
  }

  kvs::AttnParams& p = plan->p;
  p = kvs::AttnParams{};
  p.q = q->data;
  p.k = k_cache->data;
  p.v = v_cache ? v_cache->data : nullptr;
  p.table = static_cast<const int32_t*>(table->data);
  p.cu_q = cu ? static_cast<const int32_t*>(cu->data) : nullptr;
  p.lens_k = lk ? static_cast<const int32_t*>(lk->data) : nullptr;
  p.out = out ? out->data : nullptr;
  p.lse = lse ? static_cast<float*>(lse->data) : nullptr;
  p.B = (int32_t)B;
  p.T = (int32_t)T;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.MB = (int32_t)MB;
  p.NB = (int32_t)NB;
  p.G = (int32_t)(Hq / Hkv);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal = causal ? 1 : 0;
  p.window = window;
  p.kv8 = kv8 ? (k_cache->dtype == KVS_INT8 ? 2 : 1) : 0;   // 1: E4M3 codes, 2: INT8 codes
  plan->dt = q->dtype == KVS_BF16 ? kvs::DType::BF16 : kvs::DType::F32;
  plan->D = (int)D;
  plan->decode = (T == B);
  plan->ws_bytes = 0;

  if (!plan->decode) {
    // fp32: two 4-wave workgroups per CU.  bf16: two 4-wave workgroups per
    // CU, whose separate barriers let one's softmax run under the other's
    // MFMAs -- unless one KV head's K/V for the widest table row exceeds an
    // XCD's L2 (4 MiB): the token tiles of a (sequence, head group) pair then
    // re-read it from HBM, and one 8-wave workgroup per CU (a K/V tile serving
    // 8 x 32 rows instead of 4 x 32) halves those re-reads.  FP8 / INT8
    // caches: 8-wave workgroups.
    const bool wide = 16.0 * (double)MB * (double)D * 2.0 * 2.0 > (double)(4 << 20);
    p.pnw = q->dtype == KVS_BF16 && (wide || kv8) ? 8 : 4;
    p.HW = p.G % 4 == 0 ? 4 : (p.G % 2 == 0 ? 2 : 1);
    p.TPW = p.pnw / p.HW;
    p.NHG = p.Hq / p.HW;
    // cu_seqlens_q / seqlens_k ride in LDS while two workgroups still fit in
    // a CU's 160 KiB; the persistent grid (two workgroups per CU) is sized at
    // launch
    p.pgrid = 0;
    const size_t half_cu = 80 * 1024 - 256;
    p.meta_lds = kvs::prefill_lds_bytes((int)D, q->dtype == KVS_BF16, (int)B, 1) <= half_cu ? 1 : 0;
    if (B > (1 << 24)) return fail(KVS_ERR_UNSUPPORTED, "prefill batch too large");
    // items are (token tile, sequence, head group); no sequence has more than
    // ceil(T / tile) token tiles, which bounds the item count from above
    const int64_t tile_rows = 32 * (int64_t)p.TPW;
    // (rows_bound: the rows of the whole buffer when q is a view of its first
    // rows, whose sequences a wrong decode_tail statement could run past)
    const int64_t Tb = rows_bound > T ? rows_bound : T;
    const int64_t items_bound = (Tb + tile_rows - 1) / tile_rows * B * (int64_t)p.NHG;
    p.items32 = items_bound < ((int64_t)1 << 31) ? 1 : 0;
    kvs::fast_div_magic((uint32_t)p.NHG, &p.nhg_m, &p.nhg_l);
    return plan_mixed(plan, q->dtype, kv8, (int)D, B, MB);
  }

  // decode: work plan from shapes and hints only
  if (p.G > 16) return fail(KVS_ERR_UNSUPPORTED, "decode supports at most 16 query heads per KV head (got %d)", p.G);
  if (B > 8192) return fail(KVS_ERR_UNSUPPORTED, "decode supports at most 8192 sequences per call (got %lld)", (long long)B);
  int hpw = 1;
  for (int c = 8; c >= 1; --c)
    if (Hkv % c == 0) { hpw = c; break; }
  if (Hkv / hpw > 65535) return fail(KVS_ERR_UNSUPPORTED, "too many KV heads for the decode grid");
  // one resident round: 8 waves per CU on 256 CUs, one wave per KV head
  int64_t nwg = std::max<int64_t>(1, 2048 / Hkv);
  if (hints && hints->num_splits > 0) nwg = hints->num_splits;
  // a workgroup's range holds at most 2048 blocks (its table entries sit in
  // LDS); B * MB bounds the batch's blocks from above
  nwg = std::max<int64_t>(nwg, (B * MB + 2047) / 2048);
  if (nwg > (1 << 20)) return fail(KVS_ERR_UNSUPPORTED, "num_splits too large");
  p.hpw = hpw;
  p.nwg = (int32_t)nwg;
  // partial outputs are addressed with 32-bit byte offsets
  if ((double)(nwg + B) * Hq * D * sizeof(float) >= 2147483648.0)
    return fail(KVS_ERR_UNSUPPORTED, "decode partial buffer would exceed 2 GiB (num_splits %lld)", (long long)nwg);
  const int slab = kvs::decode_slab_bytes((int)D, kv8);
  // (the whole table is copied in 16-byte pieces: it must be 16-byte aligned)
  p.dsmall = B <= kvs::kDecodeSmallB && B * MB <= kvs::kDecodeSmallTbl &&
             reinterpret_cast<uintptr_t>(table->data) % 16 == 0 &&
             kvs::decode_lds_bytes((int)B, kvs::decode_tbl_ints((int)B, (int)MB, true), hpw, slab) <= kLdsBudget;
  if (kvs::decode_lds_bytes((int)B, kvs::decode_tbl_ints((int)B, (int)MB, p.dsmall), hpw, slab) > kLdsBudget)
    return fail(KVS_ERR_UNSUPPORTED, "decode batch too large for one workgroup's LDS (B=%lld)", (long long)B);
  if (nwg > 1) {
    // The counters sit at the same place for every shape: the first
    // kvs::kDecodeCounterBytes of the workspace, counter (b, g) at index
    // b * Hkv + g.  Every call leaves the ones it used at zero, so calls of
    // any shapes may follow one another on one workspace (a layout that moved
    // with the shape would meet another call's partial outputs there).
    if (B * Hkv > (int64_t)(kvs::kDecodeCounterBytes / sizeof(int32_t)))
      return fail(KVS_ERR_UNSUPPORTED, "split decode supports B * Hkv <= %zu (got %lld)",
                  kvs::kDecodeCounterBytes / sizeof(int32_t), (long long)(B * Hkv));
    const size_t slots = (size_t)nwg + B;
    plan->ws_po_off = kvs::kDecodeCounterBytes;
    plan->ws_lse_off = plan->ws_po_off + align_up(slots * Hq * D * sizeof(float), 256);
    plan->ws_bytes = plan->ws_lse_off + align_up(slots * Hq * sizeof(float), 256);
  }
  return KVS_OK;
}

// ---- scratch of the no-allocation call (attn_varlen_paged_noalloc) --------
// A file-scope device array: each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is a stand-in, not a device address): it uses the
// address hipGetSymbolAddress returns with that device current, kept per
// device.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scr_mu;
void* g_scr[kMaxDevices];

kvs_status noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(KVS_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(KVS_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scr_mu);
  if (!g_scr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(KVS_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    }
    g_scr[dev] = ptr;
  }
  *out = g_scr[dev];
  return KVS_OK;
}

// ---- grow-only scratch for the plain call (one buffer per device) ----------
// Allocated stream-ordered on the call's stream (hipMallocAsync) and zeroed
// there by the library's own kernel; a smaller buffer it replaces is freed
// stream-ordered on the same stream, after the work already queued there.
// Nothing synchronises the device.  Calls on one device that overlap in time
// share the buffer and are not allowed (documented in the header).
std::mutex g_ws_mu;
std::vector<std::pair<void*, size_t>> g_ws;

kvs_status get_plain_workspace(size_t need, hipStream_t stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(KVS_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_ws_mu);
  if ((size_t)dev >= g_ws.size()) g_ws.resize(dev + 1, {nullptr, 0});
  auto& slot = g_ws[dev];
  if (slot.second < need) {
    void* ptr = nullptr;
    hipError_t e = hipMallocAsync(&ptr, need, stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(KVS_ERR_HIP, "hipMallocAsync(%zu) for decode scratch: %s", need, hipGetErrorString(e));
    }
    // the decode counters in the scratch must start at zero; kernels leave them zero
    e = kvs::launch_zero(ptr, need, stream);
    if (e != hipSuccess) {
      (void)hipFreeAsync(ptr, stream);
      return fail(KVS_ERR_HIP, "zeroing the decode scratch: %s", hipGetErrorString(e));
    }
    if (slot.first) (void)hipFreeAsync(slot.first, stream);
    slot = {ptr, need};
  }
  *out = slot.first;
  return KVS_OK;
}

kvs_status no_fp8(const Plan& plan) {
  if (plan.p.kv8)
    return fail(KVS_ERR_INVALID, "quantized caches need their scales: use the _fp8 / _int8 calls (attn_varlen_paged_fp8_ex, attn_varlen_paged_int8_ex)");
  return KVS_OK;
}

// " sliding_window=W" or "", in a small per-thread buffer
const char* window_note(const kvs::AttnParams& p) {
  thread_local char note[32];
  if (p.window > 0) snprintf(note, sizeof note, " sliding_window=%d", p.window);
  else note[0] = 0;
  return note;
}

#ifdef KVS_DEBUG
// Debug library only: the device-resident preconditions (cu_seqlens_q,
// seqlens_k, the table entries the call reads, store slots) are checked on
// the stream before the call's kernels are enqueued; the call waits for the
// check and a violation returns KVS_ERR_INVALID with nothing else enqueued.
kvs_status debug_check(const int32_t* cu, const int32_t* lens, const int32_t* table, int64_t B, int64_t T, int MB,
                       int NB, int window, const int32_t* slots, int64_t n_slots, int64_t num_slots,
                       hipStream_t s) {
  const kvs::CheckParams v{cu, lens, table, B, T, MB, NB, window, slots, n_slots, num_slots};
  int r[4] = {0, 0, 0, 0};
  const hipError_t e = kvs::run_check(v, s, r);
  if (e != hipSuccess) return fail(KVS_ERR_HIP, "KVS_DEBUG check did not run: %s", hipGetErrorString(e));
  switch (r[0]) {
    case 0: return KVS_OK;
    case kvs::kCheckCuFirst: return fail(KVS_ERR_INVALID, "KVS_DEBUG: cu_seqlens_q[0] = %d, not 0", r[3]);
    case kvs::kCheckCuLast:
      return fail(KVS_ERR_INVALID, "KVS_DEBUG: cu_seqlens_q[B] = %d, not T = %lld", r[3], (long long)T);
    case kvs::kCheckLq:
      return fail(KVS_ERR_INVALID, "KVS_DEBUG: sequence %d has %d query rows (needs >= 1, inside [0, T))", r[1], r[3]);
    case kvs::kCheckLk:
      return fail(KVS_ERR_INVALID, "KVS_DEBUG: seqlens_k[%d] = %d (needs query rows <= it <= 16 * MB = %d)", r[1],
                  r[3], 16 * MB);
    case kvs::kCheckTable:
      return fail(KVS_ERR_INVALID, "KVS_DEBUG: block_table[%d][%d] = %d, outside [0, NB = %d)", r[1], r[2], r[3], NB);
    default:
      return fail(KVS_ERR_INVALID, "KVS_DEBUG: slot_mapping[%d] = %d, outside [0, 16 * NB = %lld)", r[1], r[3],
                  (long long)num_slots);
  }
}
#define KVS_DEBUG_CHECK(...) KVS_TRY(debug_check(__VA_ARGS__))
#else
#define KVS_DEBUG_CHECK(...) \
  do {                       \
  } while (0)
#endif

kvs_status run_plan(Plan& plan, void* ws, size_t ws_bytes, hipStream_t stream) {
  kvs::AttnParams& p = plan.p;
  KVS_DEBUG_CHECK(plan.decode ? nullptr : p.cu_q, p.lens_k, p.table, p.B, p.T, p.MB, p.NB, p.window, nullptr, 0, 0,
                  stream);
  if (plan.decode) {
    if (plan.ws_bytes) {
      if (!ws || ws_bytes < plan.ws_bytes)
        return fail(KVS_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", plan.ws_bytes, ws_bytes);
      if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(KVS_ERR_WORKSPACE, "workspace must be 256-byte aligned");
      p.counters = static_cast<int32_t*>(ws);
      p.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + plan.ws_po_off);
      p.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + plan.ws_lse_off);
    }
    const hipError_t e = kvs::launch_decode(p, plan.dt, plan.D, stream);
    if (e != hipSuccess) return fail(KVS_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    set_dispatch("decode_%s%s_d%d grid=(%d,%d) waves/wg=%d ranges=%d table=%s%s", plan.dt == kvs::DType::BF16 ? "bf16" : "f32",
                 p.kv8 ? (p.kv8 == 2 ? "_kv_int8" : "_kv_fp8") : "", plan.D, p.nwg, p.Hkv / p.hpw, p.hpw, p.nwg, p.dsmall ? "whole" : "window",
                 window_note(p));
    return KVS_OK;
  }
  if (plan.mixed) {
    if (ws && ws_bytes >= plan.ws_bytes && reinterpret_cast<uintptr_t>(ws) % 256 == 0) {
      p.counters = static_cast<int32_t*>(ws);
      p.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + plan.ws_po_off);
      p.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + plan.ws_lse_off);
      const hipError_t e = kvs::launch_mixed(p, plan.D, plan.mixed_grid, plan.mixed_lds, stream);
      if (e != hipSuccess) return fail(KVS_ERR_HIP, "mixed launch failed: %s", hipGetErrorString(e));
      set_dispatch("mixed_bf16_d%d grid=%d (prefill items of multi-row sequences | decode ranges of one-row sequences, "
                   "split in-kernel) waves/wg=%d head groups=%d heads/wg=%d tokens/item=%d%s",
                   plan.D, plan.mixed_grid, p.pnw, p.NHG, p.HW, 32 * p.TPW, window_note(p));
      return KVS_OK;
    }
    // no (or too small a) workspace: every sequence goes through the prefill kernel
    p.mixed = 0;
  }
  int cus = 0;
  KVS_TRY(device_cus(&cus));
  p.pgrid = (p.pnw == 8 ? 1 : 2) * cus;
  const hipError_t e = kvs::launch_prefill(p, plan.dt, plan.D, stream);
  if (e != hipSuccess) return fail(KVS_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  set_dispatch("prefill_%s%s_d%d grid=%d (persistent) waves/wg=%d head groups=%d heads/wg=%d tokens/item=%d meta_lds=%d%s",
               plan.dt == kvs::DType::BF16 ? "bf16" : "f32", p.kv8 ? (p.kv8 == 2 ? "_kv_int8" : "_kv_fp8") : "", plan.D, p.pgrid, p.pnw, p.NHG,
               p.HW, 32 * p.TPW, p.meta_lds, window_note(p));
  return KVS_OK;
}

}  // namespace

extern "C" {

kvs_status kv_store_paged(const kvs_tensor* k_new, const kvs_tensor* v_new, const kvs_tensor* slot_mapping,
                          kvs_tensor* k_cache, kvs_tensor* v_cache, kvs_stream_t stream) {
  clear_error();
  KVS_TRY(check_tensor(k_cache, "k_cache", kFloatTypes, 4));
  KVS_TRY(check_tensor(v_cache, "v_cache", kFloatTypes, 4));
  KVS_TRY(check_tensor(k_new, "k_new", kFloatTypes, 3, true));
  KVS_TRY(check_tensor(v_new, "v_new", kFloatTypes, 3, true));
  KVS_TRY(check_tensor(slot_mapping, "slot_mapping", kIntTypes, 1, true));
  const int64_t Tn = k_new->shape[0];
  for (int i = 0; i < 4; ++i)
    if (v_cache->shape[i] != k_cache->shape[i]) return fail(KVS_ERR_INVALID, "v_cache shape != k_cache shape");
  for (int i = 0; i < 3; ++i)
    if (v_new->shape[i] != k_new->shape[i]) return fail(KVS_ERR_INVALID, "v_new shape != k_new shape");
  if (k_cache->dtype != v_cache->dtype || k_new->dtype != k_cache->dtype || v_new->dtype != k_cache->dtype)
    return fail(KVS_ERR_INVALID, "k_new, v_new, k_cache and v_cache must share one dtype");
  if (k_cache->shape[1] != 16) return fail(KVS_ERR_UNSUPPORTED, "page size %lld not supported (only 16)", (long long)k_cache->shape[1]);
  if (k_new->shape[1] != k_cache->shape[2] || k_new->shape[2] != k_cache->shape[3])
    return fail(KVS_ERR_INVALID, "k_new [T, Hkv, D] does not match the pool's [.., .., Hkv, D]");
  if (slot_mapping->shape[0] != Tn) return fail(KVS_ERR_INVALID, "slot_mapping has %lld entries for %lld rows", (long long)slot_mapping->shape[0], (long long)Tn);
  const int64_t row_bytes = k_new->shape[1] * k_new->shape[2] * esize(k_new->dtype);
  if (row_bytes % 16) return fail(KVS_ERR_UNSUPPORTED, "token row of %lld bytes is not a multiple of 16", (long long)row_bytes);
  if (Tn == 0) {
    set_dispatch("kv_store_paged: empty (nothing enqueued)");
    return KVS_OK;
  }
  kvs::StoreParams p{};
  p.k_new = k_new->data;
  p.v_new = v_new->data;
  p.slots = static_cast<const int32_t*>(slot_mapping->data);
  p.k_cache = k_cache->data;
  p.v_cache = v_cache->data;
  p.t_new = Tn;
  p.row_chunks = row_bytes / 16;
  p.num_slots = k_cache->shape[0] * 16;
  KVS_DEBUG_CHECK(nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, p.slots, Tn, p.num_slots, reinterpret_cast<hipStream_t>(stream));
  const hipError_t e = kvs::launch_store(p, k_new->dtype == KVS_BF16 ? kvs::DType::BF16 : kvs::DType::F32,
                                         reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVS_ERR_HIP, "kv_store_paged launch failed: %s", hipGetErrorString(e));
  set_dispatch("kv_store_paged rows=%lld row_bytes=%lld", (long long)Tn, (long long)row_bytes);
  return KVS_OK;
}

// The quantizing store of kv_store_paged_fp8 / kv_store_paged_int8: `code` is
// the cache dtype (KVS_FP8_E4M3 or KVS_INT8).
static kvs_status store_q8(const kvs_tensor* k_new, const kvs_tensor* v_new, const kvs_tensor* slot_mapping,
                    kvs_tensor* k_cache, kvs_tensor* v_cache, kvs_tensor* k_scale, kvs_tensor* v_scale,
                    kvs_stream_t stream, int code) {
  const char* name = code == KVS_INT8 ? "kv_store_paged_int8" : "kv_store_paged_fp8";
  KVS_TRY(check_tensor(k_cache, "k_cache", 1u << code, 4));
  KVS_TRY(check_tensor(v_cache, "v_cache", 1u << code, 4));
  KVS_TRY(check_tensor(k_scale, "k_scale", 1u << KVS_F32, 3));
  KVS_TRY(check_tensor(v_scale, "v_scale", 1u << KVS_F32, 3));
  KVS_TRY(check_tensor(k_new, "k_new", kFloatTypes, 3, true));
  KVS_TRY(check_tensor(v_new, "v_new", kFloatTypes, 3, true));
  KVS_TRY(check_tensor(slot_mapping, "slot_mapping", kIntTypes, 1, true));
  const int64_t Tn = k_new->shape[0], NB = k_cache->shape[0], Hkv = k_cache->shape[2], D = k_cache->shape[3];
  for (int i = 0; i < 4; ++i)
    if (v_cache->shape[i] != k_cache->shape[i]) return fail(KVS_ERR_INVALID, "v_cache shape != k_cache shape");
  for (int i = 0; i < 3; ++i)
    if (v_new->shape[i] != k_new->shape[i]) return fail(KVS_ERR_INVALID, "v_new shape != k_new shape");
  if (v_new->dtype != k_new->dtype) return fail(KVS_ERR_INVALID, "v_new dtype != k_new dtype");
  if (k_cache->shape[1] != 16) return fail(KVS_ERR_UNSUPPORTED, "page size %lld not supported (only 16)", (long long)k_cache->shape[1]);
  if (D != 64 && D != 128) return fail(KVS_ERR_UNSUPPORTED, "head dim %lld not supported (64 or 128)", (long long)D);
  if (k_new->shape[1] != Hkv || k_new->shape[2] != D)
    return fail(KVS_ERR_INVALID, "k_new [T, Hkv, D] does not match the pool's [.., .., Hkv, D]");
  for (const kvs_tensor* t : {k_scale, v_scale})
    if (t->shape[0] != NB || t->shape[1] != Hkv || t->shape[2] != 16)
      return fail(KVS_ERR_INVALID, "scales must be [NB, Hkv, 16] = [%lld, %lld, 16]", (long long)NB, (long long)Hkv);
  if (slot_mapping->shape[0] != Tn) return fail(KVS_ERR_INVALID, "slot_mapping has %lld entries for %lld rows", (long long)slot_mapping->shape[0], (long long)Tn);
  if (Tn == 0) {
    set_dispatch("%s: empty (nothing enqueued)", name);
    return KVS_OK;
  }
  kvs::StoreFp8Params p{};
  p.k_new = k_new->data;
  p.v_new = v_new->data;
  p.slots = static_cast<const int32_t*>(slot_mapping->data);
  p.k_cache = k_cache->data;
  p.v_cache = v_cache->data;
  p.k_scale = static_cast<float*>(k_scale->data);
  p.v_scale = static_cast<float*>(v_scale->data);
  p.t_new = Tn;
  p.num_slots = NB * 16;
  p.Hkv = (int32_t)Hkv;
  KVS_DEBUG_CHECK(nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, p.slots, Tn, p.num_slots, reinterpret_cast<hipStream_t>(stream));
  const hipError_t e = kvs::launch_store_fp8(p, k_new->dtype == KVS_BF16 ? kvs::DType::BF16 : kvs::DType::F32, (int)D,
                                             code == KVS_INT8, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVS_ERR_HIP, "%s launch failed: %s", name, hipGetErrorString(e));
  set_dispatch("%s rows=%lld kv_heads=%lld head_dim=%lld", name, (long long)Tn, (long long)Hkv, (long long)D);
  return KVS_OK;
}

kvs_status kv_store_paged_fp8(const kvs_tensor* k_new, const kvs_tensor* v_new, const kvs_tensor* slot_mapping,
                              kvs_tensor* k_cache, kvs_tensor* v_cache, kvs_tensor* k_scale, kvs_tensor* v_scale,
                              kvs_stream_t stream) {
  clear_error();
  return store_q8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream, KVS_FP8_E4M3);
}

kvs_status kv_store_paged_int8(const kvs_tensor* k_new, const kvs_tensor* v_new, const kvs_tensor* slot_mapping,
                               kvs_tensor* k_cache, kvs_tensor* v_cache, kvs_tensor* k_scale, kvs_tensor* v_scale,
                               kvs_stream_t stream) {
  clear_error();
  return store_q8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream, KVS_INT8);
}

kvs_status kv_store_rope_paged(kvs_tensor* q, const kvs_tensor* k_new, const kvs_tensor* v_new,
                               const kvs_tensor* positions, const kvs_tensor* slot_mapping, kvs_tensor* k_cache,
                               kvs_tensor* v_cache, const kvs_rope* rope, kvs_stream_t stream) {
  clear_error();
  KVS_TRY(check_tensor(k_cache, "k_cache", kFloatTypes, 4));
  KVS_TRY(check_tensor(v_cache, "v_cache", kFloatTypes, 4));
  KVS_TRY(check_tensor(k_new, "k_new", kFloatTypes, 3, true));
  KVS_TRY(check_tensor(v_new, "v_new", kFloatTypes, 3, true));
  KVS_TRY(check_tensor(positions, "positions", kIntTypes, 1, true));
  KVS_TRY(check_tensor(slot_mapping, "slot_mapping", kIntTypes, 1, true));
  if (q) KVS_TRY(check_tensor(q, "q", kFloatTypes, 3, true));
  if (!rope) return fail(KVS_ERR_INVALID, "rope: parameters are NULL");
  const int64_t Tn = k_new->shape[0], Hkv = k_cache->shape[2], D = k_cache->shape[3];
  for (int i = 0; i < 4; ++i)
    if (v_cache->shape[i] != k_cache->shape[i]) return fail(KVS_ERR_INVALID, "v_cache shape != k_cache shape");
  for (int i = 0; i < 3; ++i)
    if (v_new->shape[i] != k_new->shape[i]) return fail(KVS_ERR_INVALID, "v_new shape != k_new shape");
  if (k_cache->dtype != v_cache->dtype || k_new->dtype != k_cache->dtype || v_new->dtype != k_cache->dtype ||
      (q && q->dtype != k_cache->dtype))
    return fail(KVS_ERR_INVALID, "q, k_new, v_new, k_cache and v_cache must share one dtype");
  if (k_cache->shape[1] != 16) return fail(KVS_ERR_UNSUPPORTED, "page size %lld not supported (only 16)", (long long)k_cache->shape[1]);
  if (k_new->shape[1] != Hkv || k_new->shape[2] != D)
    return fail(KVS_ERR_INVALID, "k_new [T, Hkv, D] does not match the pool's [.., .., Hkv, D]");
  if (q && (q->shape[0] != Tn || q->shape[2] != D || q->shape[1] < 1))
    return fail(KVS_ERR_INVALID, "q must be [T, Hq, D] with the rows and head dim of k_new");
  if (positions->shape[0] != Tn) return fail(KVS_ERR_INVALID, "positions has %lld entries for %lld rows", (long long)positions->shape[0], (long long)Tn);
  if (slot_mapping->shape[0] != Tn) return fail(KVS_ERR_INVALID, "slot_mapping has %lld entries for %lld rows", (long long)slot_mapping->shape[0], (long long)Tn);
  if (D % 16 || D > 2 * kvs::kRopeMaxPairs) return fail(KVS_ERR_UNSUPPORTED, "rope: head dim %lld not supported (a multiple of 16, at most %d)", (long long)D, 2 * kvs::kRopeMaxPairs);
  const int64_t rd = rope->rotary_dim ? rope->rotary_dim : D;
  if (rd < 16 || rd > D || rd % 16) return fail(KVS_ERR_INVALID, "rope: rotary_dim %lld must be a multiple of 16 in [16, D]", (long long)rd);
  if (rope->style != KVS_ROPE_NEOX && rope->style != KVS_ROPE_INTERLEAVED) return fail(KVS_ERR_INVALID, "rope: unknown style %d", (int)rope->style);
  if (!(std::isfinite(rope->base) && rope->base > 0) || !(std::isfinite(rope->pos_scale) && rope->pos_scale > 0))
    return fail(KVS_ERR_INVALID, "rope: base and pos_scale must be finite and positive");
  if (Tn > INT32_MAX || (q && q->shape[1] > 4096)) return fail(KVS_ERR_UNSUPPORTED, "rope: sizes beyond the kernel's ranges");
  if (Tn == 0) {
    set_dispatch("kv_store_rope_paged: empty (nothing enqueued)");
    return KVS_OK;
  }
  kvs::RopeParams p{};
  p.q = q ? q->data : nullptr;
  p.k_new = k_new->data;
  p.v_new = v_new->data;
  p.pos = static_cast<const int32_t*>(positions->data);
  p.slots = static_cast<const int32_t*>(slot_mapping->data);
  p.k_cache = k_cache->data;
  p.v_cache = v_cache->data;
  p.T = Tn;
  p.num_slots = k_cache->shape[0] * 16;
  p.Hq = q ? (int32_t)q->shape[1] : 0;
  p.Hkv = (int32_t)Hkv;
  p.D = (int32_t)D;
  p.rd = (int32_t)rd;
  p.style = rope->style;
  p.inv_scale = 1.0 / rope->pos_scale;
  for (int i = 0; i < rd / 2; ++i) p.inv_freq[i] = std::pow(rope->base, -2.0 * i / (double)rd);
  KVS_DEBUG_CHECK(nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, p.slots, Tn, p.num_slots, reinterpret_cast<hipStream_t>(stream));
  const hipError_t e = kvs::launch_rope_store(p, k_cache->dtype == KVS_BF16 ? kvs::DType::BF16 : kvs::DType::F32,
                                              reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVS_ERR_HIP, "kv_store_rope_paged launch failed: %s", hipGetErrorString(e));
  set_dispatch("kv_store_rope_paged rows=%lld q_heads=%d kv_heads=%lld rotary_dim=%lld style=%s", (long long)Tn,
               p.Hq, (long long)Hkv, (long long)rd, rope->style == KVS_ROPE_NEOX ? "neox" : "interleaved");
  return KVS_OK;
}

kvs_status attn_varlen_paged(const kvs_tensor* q, const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                             const kvs_tensor* block_table, const kvs_tensor* cu_seqlens_q,
                             const kvs_tensor* seqlens_k, float scale, int causal, kvs_tensor* out,
                             kvs_tensor* lse, kvs_stream_t stream) {
  clear_error();
  Plan plan;
  KVS_TRY(make_plan(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, scale, causal, out, lse, nullptr,
                    false, &plan));
  KVS_TRY(no_fp8(plan));
  void* ws = nullptr;
  if (plan.ws_bytes) KVS_TRY(get_plain_workspace(plan.ws_bytes, reinterpret_cast<hipStream_t>(stream), &ws));
  return run_plan(plan, ws, plan.ws_bytes, reinterpret_cast<hipStream_t>(stream));
}

kvs_status attn_varlen_paged_noalloc(const kvs_tensor* q, const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                     const kvs_tensor* block_table, const kvs_tensor* cu_seqlens_q,
                                     const kvs_tensor* seqlens_k, float scale, int causal, kvs_tensor* out,
                                     kvs_tensor* lse, kvs_stream_t stream) {
  clear_error();
  Plan plan;
  KVS_TRY(make_plan(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, scale, causal, out, lse, nullptr,
                    false, &plan));
  KVS_TRY(no_fp8(plan));
  void* ws = nullptr;
  // a mixed batch whose scratch does not fit runs in the prefill kernel alone
  if (plan.mixed && plan.ws_bytes > kNoAllocScratchBytes) return run_plan(plan, nullptr, 0, reinterpret_cast<hipStream_t>(stream));
  if (plan.ws_bytes) {
    if (plan.ws_bytes > kNoAllocScratchBytes)
      return fail(KVS_ERR_WORKSPACE,
                  "these shapes need %zu bytes of decode scratch; the no-allocation call's static scratch holds %zu "
                  "(use attn_varlen_paged_ex with a caller workspace)",
                  plan.ws_bytes, kNoAllocScratchBytes);
    KVS_TRY(noalloc_scratch(&ws));
    // the merge counters this call uses (index b * Hkv + g) must start at
    // zero: clear them on the stream with the library's own kernel
    const size_t cbytes = align_up((size_t)plan.p.B * plan.p.Hkv * sizeof(int32_t), 16);
    const hipError_t e = kvs::launch_zero(ws, cbytes, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KVS_ERR_HIP, "clearing the static scratch's counters: %s", hipGetErrorString(e));
  }
  return run_plan(plan, ws, kNoAllocScratchBytes, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

kvs_status check_hints(const kvs_hints* h);

kvs_status decode_append(const kvs_tensor* q, const kvs_tensor* k_new, const kvs_tensor* v_new,
                         kvs_tensor* k_cache, kvs_tensor* v_cache, const kvs_tensor* block_table,
                         const kvs_tensor* seqlens_k, float scale, int window, kvs_tensor* out, kvs_tensor* lse,
                         const kvs_hints* hints, void* workspace, size_t workspace_bytes, kvs_stream_t stream,
                         const kvs_rope* rope = nullptr, kvs_tensor* k_scale = nullptr,
                         kvs_tensor* v_scale = nullptr, int q8 = 1) {
  KVS_TRY(check_hints(hints));
  Plan plan;
  KVS_TRY(make_plan(q, k_cache, v_cache, block_table, nullptr, seqlens_k, scale, 1, out, lse, hints, false,
                    &plan, true, window));
  if (k_scale) {
    // FP8 cache: the new rows are quantized as kv_store_paged_fp8 does
    KVS_TRY(check_tensor(k_scale, "k_scale", 1u << KVS_F32, 3));
    KVS_TRY(check_tensor(v_scale, "v_scale", 1u << KVS_F32, 3));
    if (plan.p.kv8 != q8)
      return fail(KVS_ERR_INVALID, "k_cache / v_cache must hold %s codes here", q8 == 2 ? "INT8" : "FP8 (E4M3)");
    const int64_t NB = k_cache->shape[0], Hkv = k_cache->shape[2];
    for (const kvs_tensor* t : {k_scale, v_scale})
      if (t->shape[0] != NB || t->shape[1] != Hkv || t->shape[2] != 16)
        return fail(KVS_ERR_INVALID, "scales must be [NB, Hkv, 16] = [%lld, %lld, 16]", (long long)NB, (long long)Hkv);
    plan.p.k_scale = static_cast<const float*>(k_scale->data);
    plan.p.v_scale = static_cast<const float*>(v_scale->data);
    plan.p.k_scale_w = static_cast<float*>(k_scale->data);
    plan.p.v_scale_w = static_cast<float*>(v_scale->data);
  } else {
    KVS_TRY(no_fp8(plan));
  }
  KVS_TRY(check_tensor(k_new, "k_new", kFloatTypes, 3));
  KVS_TRY(check_tensor(v_new, "v_new", kFloatTypes, 3));
  for (int i = 0; i < 3; ++i)
    if (v_new->shape[i] != k_new->shape[i]) return fail(KVS_ERR_INVALID, "v_new shape != k_new shape");
  if (k_new->dtype != q->dtype || v_new->dtype != q->dtype) return fail(KVS_ERR_INVALID, "k_new / v_new dtype != q dtype");
  if (rope && plan.p.kv8) return fail(KVS_ERR_UNSUPPORTED, "rope with a quantized cache in the fused decode step");
  if (k_new->shape[0] != q->shape[0] || k_new->shape[1] != k_cache->shape[2] || k_new->shape[2] != k_cache->shape[3])
    return fail(KVS_ERR_INVALID, "k_new must be [B, Hkv, D] = [%lld, %lld, %lld]", (long long)q->shape[0],
                (long long)k_cache->shape[2], (long long)k_cache->shape[3]);
  kvs::AttnParams& p = plan.p;
  p.k_new = k_new->data;
  p.v_new = v_new->data;
  p.k_cache_w = k_cache->data;
  p.v_cache_w = v_cache->data;
  p.append = 1;
  if (rope) {
    // the pairs of a lane's chunks must stay in the lane: neox halves a
    // multiple of 32 dims apart, interleaved pairs inside 8-value chunks
    if (plan.dt != kvs::DType::BF16) return fail(KVS_ERR_UNSUPPORTED, "rope in the fused decode step: bf16 only");
    const int64_t D = plan.D, rd = rope->rotary_dim ? rope->rotary_dim : D;
    if (rope->style != KVS_ROPE_NEOX && rope->style != KVS_ROPE_INTERLEAVED)
      return fail(KVS_ERR_INVALID, "rope: unknown style %d", (int)rope->style);
    const int64_t step = rope->style == KVS_ROPE_NEOX ? 64 : 16;
    if (rd < step || rd > D || rd % step)
      return fail(KVS_ERR_UNSUPPORTED, "rope in the fused decode step: rotary_dim %lld must be a multiple of %lld in [%lld, D]",
                  (long long)rd, (long long)step, (long long)step);
    if (!(std::isfinite(rope->base) && rope->base > 0) || !(std::isfinite(rope->pos_scale) && rope->pos_scale > 0))
      return fail(KVS_ERR_INVALID, "rope: base and pos_scale must be finite and positive");
    p.rope = 1;
    p.rope_rd = (int32_t)rd;
    p.rope_style = rope->style;
    p.rope_inv_scale = 1.0 / rope->pos_scale;
    p.rope_l2b = std::log2(rope->base);
    // the decode LDS grows by the per-wave angle table (the whole-table set-up
    // gives way to the windowed one if both no longer fit)
    auto need = [&] {
      return kvs::decode_lds_bytes(p.B, kvs::decode_tbl_ints(p.B, p.MB, p.dsmall), p.hpw,
                                   kvs::decode_slab_bytes((int)D, false, true));
    };
    constexpr size_t kLdsBudget = 160 * 1024 - 256;
    if (p.dsmall && need() > kLdsBudget) p.dsmall = 0;
    if (need() > kLdsBudget) return fail(KVS_ERR_UNSUPPORTED, "decode batch too large for one workgroup's LDS (B=%d)", p.B);
  }
  KVS_TRY(run_plan(plan, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream)));
  set_dispatch("decode_append_%s%s_d%d grid=(%d,%d) waves/wg=%d ranges=%d table=%s%s%s",
               plan.dt == kvs::DType::BF16 ? "bf16" : "f32", p.kv8 ? (p.kv8 == 2 ? "_kv_int8" : "_kv_fp8") : "", plan.D, p.nwg, p.Hkv / p.hpw,
               p.hpw, p.nwg, p.dsmall ? "whole" : "window", window_note(p), p.rope ? " rope" : "");
  return KVS_OK;
}

// One attention call's arguments (scales only for FP8 caches).
struct AttnCall {
  const kvs_tensor *q, *k, *v, *ks, *vs, *table, *cu, *lk;
  float scale;
  int causal, window;
  kvs_tensor *out, *lse;
  const kvs_hints* hints;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  int64_t rows_bound;   // rows of the whole q when q is a row view (0: q's own)
};

kvs_status check_hints(const kvs_hints* h) {
  if (h && (h->num_splits < 0 || h->max_seqlen_k < 0 || h->max_seqlen_q < 0 || h->decode_tail < 0))
    return fail(KVS_ERR_INVALID, "hints must be non-negative");
  return KVS_OK;
}

kvs_status run_call(const AttnCall& c) {
  Plan plan;
  KVS_TRY(make_plan(c.q, c.k, c.v, c.table, c.cu, c.lk, c.scale, c.causal, c.out, c.lse, c.hints, false, &plan,
                    false, c.window, c.rows_bound));
  if (c.ks) {
    plan.p.k_scale = static_cast<const float*>(c.ks->data);
    plan.p.v_scale = static_cast<const float*>(c.vs->data);
  } else {
    KVS_TRY(no_fp8(plan));
  }
  return run_plan(plan, c.ws, c.ws_bytes, c.stream);
}

// Rows [r0, r0 + n) of a dense descriptor (a view; nothing is copied).
kvs_tensor rows_of(const kvs_tensor* t, int64_t r0, int64_t n) {
  kvs_tensor v = *t;
  int64_t row = 1;
  for (int i = 1; i < t->ndim; ++i) row *= t->shape[i];
  v.data = static_cast<char*>(t->data) + r0 * row * esize(t->dtype);
  v.shape[0] = n;
  return v;
}

// The batch split the decode_tail hint asks for: sequences [0, B - N) and
// rows [0, T - N) go to the prefill/extend path, the last N sequences -- one
// query row each, rows [T - N, T) -- to the decode path.  *n_out = 0: no
// split (the hint is absent or 0, every sequence is a decode row, or an lse
// row view would lose its 16-byte alignment; the call then runs unsplit).
kvs_status tail_split(const AttnCall& c, int64_t* n_out) {
  *n_out = 0;
  const int64_t N = c.hints ? c.hints->decode_tail : 0;
  if (N <= 0) return KVS_OK;
  KVS_TRY(check_tensor(c.q, "q", kFloatTypes, 3));
  KVS_TRY(check_tensor(c.table, "block_table", kIntTypes, 2));
  const int64_t T = c.q->shape[0], B = c.table->shape[0];
  if (N > B) return fail(KVS_ERR_INVALID, "decode_tail %lld does not fit B=%lld", (long long)N, (long long)B);
  if (N == B) {
    if (T != B)
      return fail(KVS_ERR_INVALID, "decode_tail = B needs one query row per sequence (T=%lld, B=%lld)", (long long)T,
                  (long long)B);
    return KVS_OK;
  }
  if (c.lse && ((T - N) * c.q->shape[1] * 4) % 16) return KVS_OK;
  *n_out = N;
  return KVS_OK;
}

kvs_status run_hinted(const AttnCall& c) {
  int64_t N = 0;
  KVS_TRY(tail_split(c, &N));
  if (!N) return run_call(c);
  KVS_TRY(check_tensor(c.out, "out", kFloatTypes, 3));
  KVS_TRY(check_tensor(c.cu, "cu_seqlens_q", kIntTypes, 1));
  KVS_TRY(check_tensor(c.lk, "seqlens_k", kIntTypes, 1));
  if (c.lse) KVS_TRY(check_tensor(c.lse, "lse", 1u << KVS_F32, 2));
  const int64_t T = c.q->shape[0], B = c.table->shape[0];
  if (c.out->shape[0] != T || c.cu->shape[0] != B + 1 || c.lk->shape[0] != B || (c.lse && c.lse->shape[0] != T))
    return fail(KVS_ERR_INVALID, "out, lse, cu_seqlens_q and seqlens_k must cover the T=%lld rows of B=%lld sequences",
                (long long)T, (long long)B);
  kvs_hints sub = *c.hints;
  sub.decode_tail = 0;
  const int64_t Bp = B - N, Tp = T - N;
  // prefill / extend part: the first Bp sequences
  kvs_tensor qp = rows_of(c.q, 0, Tp), op = rows_of(c.out, 0, Tp), tp = rows_of(c.table, 0, Bp);
  kvs_tensor cp = rows_of(c.cu, 0, Bp + 1), kp = rows_of(c.lk, 0, Bp);
  kvs_tensor lp = c.lse ? rows_of(c.lse, 0, Tp) : kvs_tensor{};
  AttnCall pre = c;
  pre.q = &qp; pre.out = &op; pre.table = &tp; pre.cu = &cp; pre.lk = &kp; pre.lse = c.lse ? &lp : nullptr;
  pre.hints = &sub;
  pre.rows_bound = T;
  // decode part: the last N sequences, one row each (cu_seqlens_q is not read there)
  kvs_tensor qd = rows_of(c.q, Tp, N), od = rows_of(c.out, Tp, N), td = rows_of(c.table, Bp, N);
  kvs_tensor cd = rows_of(c.cu, 0, N + 1), kd = rows_of(c.lk, Bp, N);
  kvs_tensor ld = c.lse ? rows_of(c.lse, Tp, N) : kvs_tensor{};
  AttnCall dec = c;
  dec.q = &qd; dec.out = &od; dec.table = &td; dec.cu = &cd; dec.lk = &kd; dec.lse = c.lse ? &ld : nullptr;
  dec.hints = &sub;
  KVS_TRY(run_call(pre));
  char d1[kTextBytes];
  memcpy(d1, g_dispatch, kTextBytes);
  KVS_TRY(run_call(dec));
  set_dispatch("split (decode_tail %lld): %s | %s", (long long)N, d1, g_dispatch);
  return KVS_OK;
}

}  // namespace

extern "C" {

kvs_status attn_decode_append_paged(const kvs_tensor* q, const kvs_tensor* k_new, const kvs_tensor* v_new,
                                    kvs_tensor* k_cache, kvs_tensor* v_cache, const kvs_tensor* block_table,
                                    const kvs_tensor* seqlens_k, float scale, kvs_tensor* out, kvs_tensor* lse,
                                    const kvs_hints* hints, void* workspace, size_t workspace_bytes,
                                    kvs_stream_t stream) {
  clear_error();
  return decode_append(q, k_new, v_new, k_cache, v_cache, block_table, seqlens_k, scale, 0, out, lse, hints,
                       workspace, workspace_bytes, stream);
}

kvs_status attn_decode_append_paged_fp8(const kvs_tensor* q, const kvs_tensor* k_new, const kvs_tensor* v_new,
                                        kvs_tensor* k_cache, kvs_tensor* v_cache, kvs_tensor* k_scale,
                                        kvs_tensor* v_scale, const kvs_tensor* block_table,
                                        const kvs_tensor* seqlens_k, float scale, int32_t window, kvs_tensor* out,
                                        kvs_tensor* lse, const kvs_hints* hints, void* workspace,
                                        size_t workspace_bytes, kvs_stream_t stream) {
  clear_error();
  if (window < 0) return fail(KVS_ERR_INVALID, "window must be >= 0 (0: none)");
  if (!k_scale || !v_scale) return fail(KVS_ERR_INVALID, "k_scale / v_scale: descriptor is NULL");
  return decode_append(q, k_new, v_new, k_cache, v_cache, block_table, seqlens_k, scale, window, out, lse, hints,
                       workspace, workspace_bytes, stream, nullptr, k_scale, v_scale);
}

kvs_status attn_decode_append_paged_int8(const kvs_tensor* q, const kvs_tensor* k_new, const kvs_tensor* v_new,
                                         kvs_tensor* k_cache, kvs_tensor* v_cache, kvs_tensor* k_scale,
                                         kvs_tensor* v_scale, const kvs_tensor* block_table,
                                         const kvs_tensor* seqlens_k, float scale, int32_t window, kvs_tensor* out,
                                         kvs_tensor* lse, const kvs_hints* hints, void* workspace,
                                         size_t workspace_bytes, kvs_stream_t stream) {
  clear_error();
  if (window < 0) return fail(KVS_ERR_INVALID, "window must be >= 0 (0: none)");
  if (!k_scale || !v_scale) return fail(KVS_ERR_INVALID, "k_scale / v_scale: descriptor is NULL");
  return decode_append(q, k_new, v_new, k_cache, v_cache, block_table, seqlens_k, scale, window, out, lse, hints,
                       workspace, workspace_bytes, stream, nullptr, k_scale, v_scale, 2);
}

kvs_status attn_decode_append_paged_rope(const kvs_tensor* q, const kvs_tensor* k_new, const kvs_tensor* v_new,
                                         kvs_tensor* k_cache, kvs_tensor* v_cache, const kvs_tensor* block_table,
                                         const kvs_tensor* seqlens_k, float scale, int32_t window, const kvs_rope* rope,
                                         kvs_tensor* out, kvs_tensor* lse, const kvs_hints* hints, void* workspace,
                                         size_t workspace_bytes, kvs_stream_t stream) {
  clear_error();
  if (window < 0) return fail(KVS_ERR_INVALID, "window must be >= 0 (0: none)");
  if (!rope) return fail(KVS_ERR_INVALID, "rope: parameters are NULL");
  return decode_append(q, k_new, v_new, k_cache, v_cache, block_table, seqlens_k, scale, window, out, lse, hints,
                       workspace, workspace_bytes, stream, rope);
}

kvs_status attn_decode_append_paged_window(const kvs_tensor* q, const kvs_tensor* k_new, const kvs_tensor* v_new,
                                           kvs_tensor* k_cache, kvs_tensor* v_cache, const kvs_tensor* block_table,
                                           const kvs_tensor* seqlens_k, float scale, int32_t window, kvs_tensor* out,
                                           kvs_tensor* lse, const kvs_hints* hints, void* workspace,
                                           size_t workspace_bytes, kvs_stream_t stream) {
  clear_error();
  if (window < 1) return fail(KVS_ERR_INVALID, "window must be >= 1 (got %d)", (int)window);
  return decode_append(q, k_new, v_new, k_cache, v_cache, block_table, seqlens_k, scale, window, out, lse, hints,
                       workspace, workspace_bytes, stream);
}

kvs_status attn_varlen_paged_ex(const kvs_tensor* q, const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                const kvs_tensor* block_table, const kvs_tensor* cu_seqlens_q,
                                const kvs_tensor* seqlens_k, float scale, int causal, kvs_tensor* out,
                                kvs_tensor* lse, const kvs_hints* hints, void* workspace,
                                size_t workspace_bytes, kvs_stream_t stream) {
  clear_error();
  KVS_TRY(check_hints(hints));
  return run_hinted(AttnCall{q, k_cache, v_cache, nullptr, nullptr, block_table, cu_seqlens_q, seqlens_k, scale,
                             causal, 0, out, lse, hints, workspace, workspace_bytes,
                             reinterpret_cast<hipStream_t>(stream)});
}

static kvs_status varlen_q8(const kvs_tensor* q, const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                            const kvs_tensor* k_scale, const kvs_tensor* v_scale, const kvs_tensor* block_table,
                            const kvs_tensor* cu_seqlens_q, const kvs_tensor* seqlens_k, float scale, int causal,
                            int32_t window, kvs_tensor* out, kvs_tensor* lse, const kvs_hints* hints, void* workspace,
                            size_t workspace_bytes, kvs_stream_t stream, int code) {
  KVS_TRY(check_hints(hints));
  if (window < 0) return fail(KVS_ERR_INVALID, "window must be >= 0 (0: none)");
  KVS_TRY(check_tensor(k_cache, "k_cache", 1u << code, 4));
  KVS_TRY(check_tensor(k_scale, "k_scale", 1u << KVS_F32, 3));
  KVS_TRY(check_tensor(v_scale, "v_scale", 1u << KVS_F32, 3));
  const int64_t NB = k_cache->shape[0], Hkv = k_cache->shape[2];
  for (const kvs_tensor* t : {k_scale, v_scale})
    if (t->shape[0] != NB || t->shape[1] != Hkv || t->shape[2] != 16)
      return fail(KVS_ERR_INVALID, "scales must be [NB, Hkv, 16] = [%lld, %lld, 16]", (long long)NB, (long long)Hkv);
  return run_hinted(AttnCall{q, k_cache, v_cache, k_scale, v_scale, block_table, cu_seqlens_q, seqlens_k, scale,
                             causal, window, out, lse, hints, workspace, workspace_bytes,
                             reinterpret_cast<hipStream_t>(stream)});
}

kvs_status attn_varlen_paged_fp8_ex(const kvs_tensor* q, const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                    const kvs_tensor* k_scale, const kvs_tensor* v_scale,
                                    const kvs_tensor* block_table, const kvs_tensor* cu_seqlens_q,
                                    const kvs_tensor* seqlens_k, float scale, int causal, int32_t window,
                                    kvs_tensor* out, kvs_tensor* lse, const kvs_hints* hints, void* workspace,
                                    size_t workspace_bytes, kvs_stream_t stream) {
  clear_error();
  return varlen_q8(q, k_cache, v_cache, k_scale, v_scale, block_table, cu_seqlens_q, seqlens_k, scale, causal, window,
                   out, lse, hints, workspace, workspace_bytes, stream, KVS_FP8_E4M3);
}

kvs_status attn_varlen_paged_int8_ex(const kvs_tensor* q, const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                     const kvs_tensor* k_scale, const kvs_tensor* v_scale,
                                     const kvs_tensor* block_table, const kvs_tensor* cu_seqlens_q,
                                     const kvs_tensor* seqlens_k, float scale, int causal, int32_t window,
                                     kvs_tensor* out, kvs_tensor* lse, const kvs_hints* hints, void* workspace,
                                     size_t workspace_bytes, kvs_stream_t stream) {
  clear_error();
  return varlen_q8(q, k_cache, v_cache, k_scale, v_scale, block_table, cu_seqlens_q, seqlens_k, scale, causal, window,
                   out, lse, hints, workspace, workspace_bytes, stream, KVS_INT8);
}

kvs_status attn_varlen_paged_window_ex(const kvs_tensor* q, const kvs_tensor* k_cache, const kvs_tensor* v_cache,
                                       const kvs_tensor* block_table, const kvs_tensor* cu_seqlens_q,
                                       const kvs_tensor* seqlens_k, float scale, int32_t window, kvs_tensor* out,
                                       kvs_tensor* lse, const kvs_hints* hints, void* workspace,
                                       size_t workspace_bytes, kvs_stream_t stream) {
  clear_error();
  KVS_TRY(check_hints(hints));
  if (window < 1) return fail(KVS_ERR_INVALID, "window must be >= 1 (got %d)", (int)window);
  return run_hinted(AttnCall{q, k_cache, v_cache, nullptr, nullptr, block_table, cu_seqlens_q, seqlens_k, scale, 1,
                             window, out, lse, hints, workspace, workspace_bytes,
                             reinterpret_cast<hipStream_t>(stream)});
}

size_t attn_varlen_paged_workspace_size(const kvs_tensor* q, const kvs_tensor* k_cache,
                                        const kvs_tensor* block_table, const kvs_hints* hints) {
  clear_error();
  if (check_hints(hints) != KVS_OK) return (size_t)-1;
  // with the decode_tail hint only the decode part (the last N sequences,
  // one row each) needs scratch
  const AttnCall c{q, k_cache, nullptr, nullptr, nullptr, block_table, nullptr, nullptr, 1.0f, 1, 0, nullptr, nullptr,
                   hints, nullptr, 0, nullptr};
  int64_t N = 0;
  if (tail_split(c, &N) != KVS_OK) return (size_t)-1;
  kvs_tensor qd, td;
  if (N) {
    qd = rows_of(q, q->shape[0] - N, N);
    td = rows_of(block_table, block_table->shape[0] - N, N);
    q = &qd;
    block_table = &td;
  }
  Plan plan;
  if (make_plan(q, k_cache, nullptr, block_table, nullptr, nullptr, 1.0f, 1, nullptr, nullptr, hints, true,
                &plan) != KVS_OK)
    return (size_t)-1;
  return plan.ws_bytes;
}

const char* kvs_last_error(void) { return g_err; }

const char* kvs_last_dispatch(void) { return g_dispatch; }

kvs_status kvs_release_workspace(void) {
  clear_error();
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(KVS_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_ws_mu);
  if ((size_t)dev < g_ws.size() && g_ws[dev].first) {
    // the buffer may still be read by work queued on any stream of the device
    if (hipDeviceSynchronize() != hipSuccess) return fail(KVS_ERR_HIP, "hipDeviceSynchronize failed");
    const hipError_t e = hipFreeAsync(g_ws[dev].first, nullptr);
    g_ws[dev] = {nullptr, 0};
    if (e != hipSuccess || hipStreamSynchronize(nullptr) != hipSuccess)
      return fail(KVS_ERR_HIP, "freeing the decode scratch failed");
  }
  return KVS_OK;
}

}  // extern "C"
