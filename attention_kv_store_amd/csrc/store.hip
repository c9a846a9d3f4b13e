// kv_store_paged: scatter new K/V token rows into their pool slots.
//
// The store step sits right before attention in a layer's step list
// (Transformer 추론 커널 (3/10), §2) and the decode path appends each new
// token's K/V to the paged cache (tiny-vLLM series, entry 5).  A slot names one
// token row of the [NB, 16, Hkv, D] pool, so the row of all Hkv heads is one
// contiguous run of Hkv*D elements in both source and destination: the kernel
// is a row-granular copy with 16-byte lanes (HBM-bound; no arithmetic).
#include <type_traits>

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

// Zero-fill of a device buffer on a stream (bytes a multiple of 16): the
// library's own kernel, so that clearing scratch memory is a kernel node when
// a caller captures the stream into a graph.
__global__ __launch_bounds__(256) void zero_kernel(u32x4* p, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) st16(p + i, u32x4{0, 0, 0, 0});
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t want = (n16 + 255) / 256;
  const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

}  // namespace kvs

// ---- FP8 (E4M3) / INT8 store: quantize each (row, KV head) with its own scale
// A 16-lane group takes one token row of one KV head (K or V): its absmax by
// a 16-lane max, s = absmax / 448 (FP8) or absmax / 127 (INT8) and the codes
// of x / s, both divisions in fp32 and correctly rounded; the codes go to the
// row's slot, s to the [NB, Hkv, 16] scale pool.
namespace kvs {

template <bool BF16, int D, bool I8 = false>
__global__ __launch_bounds__(256) void kv_store_fp8_kernel(StoreFp8Params p) {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int EPL = D / 16;                           // values per lane: 16 lanes per row
  const int64_t gid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  if (gid >= p.t_new * p.Hkv * 2) return;               // whole 16-lane groups
  const int which = (int)(gid & 1);                     // 0: K, 1: V
  const int64_t th = gid >> 1;
  const int h = (int)(th % p.Hkv);
  const int64_t t = th / p.Hkv;
  const int32_t slot = p.slots[t];
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;  // whole group
  const E* src = static_cast<const E*>(which ? p.v_new : p.k_new) + (t * p.Hkv + h) * D + sub * EPL;
  float x[EPL];
  if constexpr (BF16) {
    uint32_t w[EPL / 2];                                // EPL bf16 values: 8 or 16 bytes
    if constexpr (EPL == 8) {
      const u32x4 v = ld16(src);
      for (int i = 0; i < 4; ++i) w[i] = v[i];
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(src);
      for (int i = 0; i < 2; ++i) w[i] = v[i];
    }
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) {
      x[2 * i] = bf16lo_to_f32(w[i]);
      x[2 * i + 1] = bf16hi_to_f32(w[i]);
    }
  } else {
#pragma unroll
    for (int c = 0; c < EPL / 4; ++c) {
      const u32x4 v = ld16(src + c * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[c * 4 + i] = __uint_as_float(v[i]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
  const float s = amax / (I8 ? 127.f : 448.f);          // correctly rounded fp32 division
  uint32_t packed[EPL / 4];
#pragma unroll
  for (int q = 0; q < EPL / 4; ++q) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w |= (s > 0.f ? (I8 ? i8_code(x[4 * q + i] / s) : e4m3_code(x[4 * q + i] / s)) : 0u) << (8 * i);
    packed[q] = w;
  }
  uint8_t* dst = static_cast<uint8_t*>(which ? p.v_cache : p.k_cache) + ((int64_t)slot * p.Hkv + h) * D + sub * EPL;
  if constexpr (EPL == 8) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{packed[0], packed[1]};
  } else {
    *reinterpret_cast<uint32_t*>(dst) = packed[0];
  }
  if (sub == 0) {
    float* sc = which ? p.v_scale : p.k_scale;
    sc[((int64_t)(slot >> 4) * p.Hkv + h) * kPage + (slot & 15)] = s;
  }
}

template <bool I8>
static void launch_store_q8(const StoreFp8Params& p, DType in, int D, dim3 g, hipStream_t s) {
  if (in == DType::BF16) {
    if (D == 64) hipLaunchKernelGGL((kv_store_fp8_kernel<true, 64, I8>), g, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((kv_store_fp8_kernel<true, 128, I8>), g, dim3(256), 0, s, p);
  } else {
    if (D == 64) hipLaunchKernelGGL((kv_store_fp8_kernel<false, 64, I8>), g, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((kv_store_fp8_kernel<false, 128, I8>), g, dim3(256), 0, s, p);
  }
}

hipError_t launch_store_fp8(const StoreFp8Params& p, DType in, int D, bool i8, hipStream_t s) {
  const int64_t threads = p.t_new * p.Hkv * 2 * 16;
  if (threads == 0) return hipSuccess;
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid);
  if (i8) launch_store_q8<true>(p, in, D, g, s);
  else launch_store_q8<false>(p, in, D, g, s);
  return hipGetLastError();
}

}  // namespace kvs
