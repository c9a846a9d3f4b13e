// kv_store_paged: scatter new K/V token rows into their pool slots.
//
// The store step sits right before attention in a layer's step list
// (Transformer 추론 커널 (3/10), §2) and the decode path appends each new
// token's K/V to the paged cache (tiny-vLLM series, entry 5).  A slot names one
// token row of the [NB, 16, Hkv, D] pool, so the row of all Hkv heads is one
// contiguous run of Hkv*D elements in both source and destination: the kernel
// is a row-granular copy with 16-byte lanes (HBM-bound; no arithmetic).
#include "kvs_device.hpp"
#include "kvs_internal.hpp"

namespace kvs {

// One lane moves one 16-byte chunk of K and the matching chunk of V.
__global__ __launch_bounds__(256) void kv_store_kernel(StoreParams p) {
  const int64_t total = p.t_new * p.row_chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t t = i / p.row_chunks;
    const int64_t c = i - t * p.row_chunks;
    const int32_t slot = p.slots[t];
    if (slot < 0) continue;  // a padding row owns no slot
    const int64_t src = t * p.row_chunks + c;
    const int64_t dst = (int64_t)slot * p.row_chunks + c;
    const u32x4 kv = ld16(static_cast<const u32x4*>(p.k_new) + src);
    const u32x4 vv = ld16(static_cast<const u32x4*>(p.v_new) + src);
    st16(static_cast<u32x4*>(p.k_cache) + dst, kv);
    st16(static_cast<u32x4*>(p.v_cache) + dst, vv);
  }
}

hipError_t launch_store(const StoreParams& p, DType, hipStream_t s) {
  const int64_t total = p.t_new * p.row_chunks;
  if (total == 0) return hipSuccess;
  // enough workgroups to fill 256 CUs several times over; grid-stride beyond
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(kv_store_kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvs
