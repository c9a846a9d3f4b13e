// Launchers of the prefill / extend kernel (prefill_impl.hpp): one
// instantiation per element type, head dim, workgroup size, sliding window and
// cache code format.
#include <atomic>

#include "prefill_impl.hpp"

namespace kvs {

template <int D, bool BF16, int NW, bool WIN, bool KV8 = false, bool I8 = false>
static hipError_t launch_prefill_t(const AttnParams& p, hipStream_t s) {
  static_assert(!I8 || (BF16 && KV8 && NW == 8), "INT8 caches: bf16 queries, 8-wave workgroups");
  const void* kern = reinterpret_cast<const void*>(&prefill_kernel<D, BF16, NW, WIN, KV8, I8>);
  const size_t lds = prefill_lds_bytes(D, BF16, p.B, p.meta_lds);
  // dynamic LDS above the default limit must be requested; grow it as needed
  // (per instantiation; atomic so that concurrent first calls are safe)
  static std::atomic<size_t> lds_granted{0};
  if (lds > lds_granted.load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // do not leave the error for the caller's next HIP call
      return e;
    }
    size_t cur = lds_granted.load(std::memory_order_relaxed);
    while (cur < lds && !lds_granted.compare_exchange_weak(cur, lds, std::memory_order_relaxed)) {
    }
  }
  hipLaunchKernelGGL((prefill_kernel<D, BF16, NW, WIN, KV8, I8>), dim3(p.pgrid), dim3(64 * NW), lds, s, p);
  return hipGetLastError();
}

template <bool WIN>
static hipError_t launch_prefill_w(const AttnParams& p, DType dt, int D, hipStream_t s) {
  if (dt == DType::BF16) {
    if (p.pnw == 8) return D == 64 ? launch_prefill_t<64, true, 8, WIN>(p, s) : launch_prefill_t<128, true, 8, WIN>(p, s);
    return D == 64 ? launch_prefill_t<64, true, 4, WIN>(p, s) : launch_prefill_t<128, true, 4, WIN>(p, s);
  }
  return D == 64 ? launch_prefill_t<64, false, 4, WIN>(p, s) : launch_prefill_t<128, false, 4, WIN>(p, s);
}

hipError_t launch_prefill(const AttnParams& p, DType dt, int D, hipStream_t s) {
  if (p.kv8 == 2) {   // INT8 caches: bf16 queries, 8-wave workgroups
    if (p.pnw != 8) return hipErrorInvalidValue;
    if (p.window > 0) return D == 64 ? launch_prefill_t<64, true, 8, true, true, true>(p, s) : launch_prefill_t<128, true, 8, true, true, true>(p, s);
    return D == 64 ? launch_prefill_t<64, true, 8, false, true, true>(p, s) : launch_prefill_t<128, true, 8, false, true, true>(p, s);
  }
  if (p.kv8) {   // FP8 caches: bf16 queries, 8-wave workgroups
    if (p.pnw != 8) return hipErrorInvalidValue;
    if (p.window > 0) return D == 64 ? launch_prefill_t<64, true, 8, true, true>(p, s) : launch_prefill_t<128, true, 8, true, true>(p, s);
    return D == 64 ? launch_prefill_t<64, true, 8, false, true>(p, s) : launch_prefill_t<128, true, 8, false, true>(p, s);
  }
  return p.window > 0 ? launch_prefill_w<true>(p, dt, D, s) : launch_prefill_w<false>(p, dt, D, s);
}

}  // namespace kvs
