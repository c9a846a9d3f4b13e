// Device calibration used by the benchmark (libkvstore_calib.so; not part of
// the attention path):
// the bf16 MFMA throughput this GPU actually sustains, to set beside the
// published peak when an attention kernel's MFMA fraction is reported.
//
// Every wave keeps four independent 32x32x16 bf16 MFMA accumulation chains
// busy for `iters` rounds (no memory traffic inside the loop), and the sum of
// its accumulators is stored once so the work cannot be dropped.
#include <hip/hip_runtime.h>

#include "../../include/kvstore_calib.h"
#include "kvs_device.hpp"

namespace kvs {

__global__ __launch_bounds__(256) void mfma_peak_kernel(const uint32_t* __restrict__ src, float* __restrict__ dst,
                                                        int iters) {
  const int lane = threadIdx.x & 63;
  const u32x4 a = ld16(src + 4 * (lane & 15));
  const u32x4 b = ld16(src + 64 + 4 * (lane & 15));
  f32x16 c0{}, c1{}, c2{}, c3{};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32x32x16_bf16(a, b, c0);
    c1 = mfma32x32x16_bf16(b, a, c1);
    c2 = mfma32x32x16_bf16(a, a, c2);
    c3 = mfma32x32x16_bf16(b, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  dst[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace kvs

extern "C" kvs_status kvs_mfma_peak_launch(const void* src, void* dst, int workgroups, int iters,
                                           kvs_stream_t stream) {
  if (!src || !dst || workgroups < 1 || iters < 1 || (reinterpret_cast<uintptr_t>(src) & 15))
    return KVS_ERR_INVALID;
  hipLaunchKernelGGL(kvs::mfma_peak_kernel, dim3(workgroups), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint32_t*>(src), static_cast<float*>(dst), iters);
  return hipGetLastError() == hipSuccess ? KVS_OK : KVS_ERR_HIP;
}
