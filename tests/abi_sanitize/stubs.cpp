// Host-only stand-ins for what the C-ABI code (csrc/api.hip) calls outside
// itself: the kernel launchers and the HIP runtime functions it uses.  Linked
// with the ABI object built under AddressSanitizer / UndefinedBehaviorSanitizer,
// they let every entry point run to completion on a machine without a GPU,
// so the sanitizers see the host-side validation and planning code.  The
// launchers check what the planner handed them instead of launching.
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>

#include "../../attention_kv_store_amd/csrc/kvs_internal.hpp"

static void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "planner handed a launcher an inconsistent plan: %s\n", what);
    std::abort();
  }
}

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 256;
  return hipSuccess;
}
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMallocAsync(void** p, size_t n, hipStream_t) {
  *p = std::aligned_alloc(256, (n + 255) / 256 * 256);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFreeAsync(void* p, hipStream_t) {
  std::free(p);
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "host stub"; }
// a device variable's address: its host shadow stands in for it here
hipError_t hipGetSymbolAddress(void** p, const void* symbol) {
  *p = const_cast<void*>(symbol);
  return hipSuccess;
}
// the module registration the compiler emits for a source with device code
static void* g_module = nullptr;
void** __hipRegisterFatBinary(const void*) { return &g_module; }
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}
void __hipUnregisterFatBinary(void**) {}
}

namespace kvs {
hipError_t launch_store(const StoreParams& p, DType, hipStream_t) {
  require(p.t_new > 0 && p.row_chunks > 0 && p.k_new && p.v_new && p.slots && p.k_cache && p.v_cache, "store");
  return hipSuccess;
}
hipError_t launch_zero(void* p, size_t bytes, hipStream_t) {
  require(p && bytes % 16 == 0, "zero");
  // the stand-in scratch is host memory: clear it as the kernel would
  for (size_t i = 0; i < bytes; ++i) static_cast<unsigned char*>(p)[i] = 0;
  return hipSuccess;
}
hipError_t launch_rope_store(const RopeParams& p, DType, hipStream_t) {
  require(p.T > 0 && p.rd >= 16 && p.rd <= p.D && p.rd % 16 == 0, "rope");
  return hipSuccess;
}
hipError_t launch_store_fp8(const StoreFp8Params& p, DType, int D, bool, hipStream_t) {
  require(p.t_new > 0 && (D == 64 || D == 128) && p.Hkv > 0, "store_fp8");
  return hipSuccess;
}
hipError_t launch_prefill(const AttnParams& p, DType, int D, hipStream_t) {
  require(p.B >= 1 && p.T >= p.B && (D == 64 || D == 128), "prefill shape");
  require(p.HW >= 1 && p.G % p.HW == 0 && p.HW * p.TPW == p.pnw && p.NHG * p.HW == p.Hq && p.pgrid > 0, "prefill map");
  require(p.q && p.k && p.v && p.table && p.cu_q && p.lens_k && p.out, "prefill pointers");
  return hipSuccess;
}
hipError_t launch_decode(const AttnParams& p, DType, int D, hipStream_t) {
  require(p.B >= 1 && p.T == p.B && (D == 64 || D == 128) && p.G <= 16, "decode shape");
  require(p.nwg >= 1 && p.hpw >= 1 && p.Hkv % p.hpw == 0, "decode map");
  require(p.nwg == 1 || (p.counters && p.part_o && p.part_lse), "decode workspace");
  return hipSuccess;
}
hipError_t launch_mixed(const AttnParams& p, int D, int grid, size_t lds, hipStream_t) {
  require(p.mixed == 1 && p.B >= 1 && p.T > p.B && (D == 64 || D == 128) && p.G <= 16, "mixed shape");
  require((p.pnw == 4 || p.pnw == 8) && p.hpw == p.pnw && p.Hkv % p.pnw == 0 && p.NHG * p.HW == p.Hq, "mixed map");
  require(grid >= 8 && grid % 8 == 0 && grid <= p.nwg && lds > 0 && lds <= 160 * 1024, "mixed grid");
  require(p.counters && p.part_o && p.part_lse && p.cu_q && p.lens_k, "mixed workspace");
  return hipSuccess;
}
hipError_t run_check(const CheckParams&, hipStream_t, int out[4]) {
  out[0] = out[1] = out[2] = out[3] = 0;
  return hipSuccess;
}
}  // namespace kvs
