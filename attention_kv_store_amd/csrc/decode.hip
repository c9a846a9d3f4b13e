// Launchers of the decode kernel (decode_impl.hpp): one instantiation per
// element type, head dim, fused append, sliding window, cache code format and
// RoPE.
#include <atomic>

#include "decode_impl.hpp"

namespace kvs {

template <int D, bool BF16, bool APPEND, bool WIN, bool KV8 = false, bool ROPE = false, bool I8 = false>
static hipError_t launch_decode_t(const AttnParams& p, hipStream_t s) {
  static_assert(!I8 || (BF16 && KV8 && !ROPE), "INT8 caches: bf16 queries");
  const void* kern = reinterpret_cast<const void*>(&decode_kernel<D, BF16, APPEND, WIN, KV8, ROPE, I8>);
  using C = DCfg<D, KV8 ? kDecodeKv8Blocks : 1>;
  static_assert(C::SLAB + (ROPE ? 2 * kRopeLdsPairs * 4 : 0) == decode_slab_bytes(D, KV8, ROPE),
                "decode_slab_bytes must match the slab layout");
  const size_t lds = decode_lds_bytes(p.B, decode_tbl_ints(p.B, p.MB, p.dsmall != 0), p.hpw,
                                      decode_slab_bytes(D, KV8, ROPE));
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
  hipLaunchKernelGGL((decode_kernel<D, BF16, APPEND, WIN, KV8, ROPE, I8>), dim3(p.nwg, p.Hkv / p.hpw), dim3(64 * p.hpw), lds, s, p);
  return hipGetLastError();
}

template <bool APPEND, bool WIN>
static hipError_t launch_decode_a(const AttnParams& p, DType dt, int D, hipStream_t s) {
  if (dt == DType::BF16)
    return D == 64 ? launch_decode_t<64, true, APPEND, WIN>(p, s) : launch_decode_t<128, true, APPEND, WIN>(p, s);
  return D == 64 ? launch_decode_t<64, false, APPEND, WIN>(p, s) : launch_decode_t<128, false, APPEND, WIN>(p, s);
}

#ifdef KVS_PHASE_TIMES
// the phase timestamps of the last decode launches (KVS_PHASE_TIMES build):
// copy out the [4096][16] array of 64-bit clock values, or clear it
extern "C" int kvs_phase_times(void* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_t), sizeof(g_phase_t), 0, hipMemcpyDeviceToHost);
}
extern "C" int kvs_phase_clear(void) {
  static unsigned long long zero[4096][kPhaseSlots];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_phase_t), zero, sizeof(zero), 0, hipMemcpyHostToDevice);
}
#endif

hipError_t launch_decode(const AttnParams& p, DType dt, int D, hipStream_t s) {
  if (p.rope) {   // fused decode step with RoPE: bf16 only
    if (dt != DType::BF16 || !p.append) return hipErrorInvalidValue;
    if (p.window > 0) return D == 64 ? launch_decode_t<64, true, true, true, false, true>(p, s) : launch_decode_t<128, true, true, true, false, true>(p, s);
    return D == 64 ? launch_decode_t<64, true, true, false, false, true>(p, s) : launch_decode_t<128, true, true, false, false, true>(p, s);
  }
  if (p.kv8 == 2) {   // INT8 caches, bf16 queries
    if (p.append) {   // the fused step
      if (p.window > 0) return D == 64 ? launch_decode_t<64, true, true, true, true, false, true>(p, s) : launch_decode_t<128, true, true, true, true, false, true>(p, s);
      return D == 64 ? launch_decode_t<64, true, true, false, true, false, true>(p, s) : launch_decode_t<128, true, true, false, true, false, true>(p, s);
    }
    if (p.window > 0) return D == 64 ? launch_decode_t<64, true, false, true, true, false, true>(p, s) : launch_decode_t<128, true, false, true, true, false, true>(p, s);
    return D == 64 ? launch_decode_t<64, true, false, false, true, false, true>(p, s) : launch_decode_t<128, true, false, false, true, false, true>(p, s);
  }
  if (p.kv8) {   // FP8 caches, bf16 queries
    if (p.append) {   // the fused step
      if (p.window > 0) return D == 64 ? launch_decode_t<64, true, true, true, true>(p, s) : launch_decode_t<128, true, true, true, true>(p, s);
      return D == 64 ? launch_decode_t<64, true, true, false, true>(p, s) : launch_decode_t<128, true, true, false, true>(p, s);
    }
    if (p.window > 0) return D == 64 ? launch_decode_t<64, true, false, true, true>(p, s) : launch_decode_t<128, true, false, true, true>(p, s);
    return D == 64 ? launch_decode_t<64, true, false, false, true>(p, s) : launch_decode_t<128, true, false, false, true>(p, s);
  }
  if (p.window > 0) return p.append ? launch_decode_a<true, true>(p, dt, D, s) : launch_decode_a<false, true>(p, dt, D, s);
  return p.append ? launch_decode_a<true, false>(p, dt, D, s) : launch_decode_a<false, false>(p, dt, D, s);
}

}  // namespace kvs
