// Device-side check of the preconditions the host cannot see without a
// synchronisation (cu_seqlens_q, seqlens_k, the block-table entries a call
// reads, store slots).  Linked only into the debug library (built with
// KVS_DEBUG), whose calls run it before their kernels, wait for it and
// return KVS_ERR_INVALID on the first violation instead of launching.  Every
// read here stays inside the arrays whose shapes the host has checked.
#include <hip/hip_runtime.h>

#include "kvs_internal.hpp"

namespace kvs {

// [0] violation code (0: none), [1] sequence or row, [2] block index, [3] value
__device__ int g_kvs_check[4];

__device__ __forceinline__ void report(int code, int where, int j, int value) {
  if (atomicCAS(&g_kvs_check[0], 0, code) == 0) {
    g_kvs_check[1] = where;
    g_kvs_check[2] = j;
    g_kvs_check[3] = value;
  }
}

// One workgroup per sequence (grid-stride): the sequence's bounds from one
// lane, then the table entries it reads from all lanes.
__global__ __launch_bounds__(256) void validate_kernel(CheckParams v) {
  for (int64_t b = blockIdx.x; b < v.B; b += gridDim.x) {
    int q0 = (int)b, q1 = (int)b + 1;   // decode: one query row per sequence
    if (v.cu_q) {
      q0 = v.cu_q[b];
      q1 = v.cu_q[b + 1];
    }
    const int lk = v.lens_k[b], lq = q1 - q0;
    if (threadIdx.x == 0) {
      if (b == 0 && q0 != 0) report(kCheckCuFirst, (int)b, 0, q0);
      if (b == v.B - 1 && q1 != v.T) report(kCheckCuLast, (int)b, 0, q1);
      if (lq < 1 || q0 < 0 || q1 > v.T) report(kCheckLq, (int)b, 0, lq);
      if (lk < lq || lk > 16 * v.MB) report(kCheckLk, (int)b, 0, lk);
    }
    if (lk < 1 || lk > 16 * v.MB || lq < 1 || lk < lq) continue;
    // blocks read: from the one holding the first row's window start (0
    // without a window) to the one holding key lk - 1
    const int first = v.window > 0 ? max(0, lk - lq - v.window + 1) >> 4 : 0;
    const int nb = (lk + 15) >> 4;
    for (int j = first + (int)threadIdx.x; j < nb; j += blockDim.x) {
      const int e = v.table[b * v.MB + j];
      if (e < 0 || e >= v.NB) report(kCheckTable, (int)b, j, e);
    }
  }
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < v.n_slots; t += stride) {
    const int s = v.slots[t];
    if (s >= 0 && (int64_t)s >= v.num_slots) report(kCheckSlot, (int)t, 0, s);
  }
}

// Runs the check on `s`, waits for it and returns its result (clearing it).
hipError_t run_check(const CheckParams& v, hipStream_t s, int out[4]) {
  const int zero[4] = {0, 0, 0, 0};
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_kvs_check), zero, sizeof(zero), 0, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  const int64_t work = v.B > (v.n_slots + 255) / 256 ? v.B : (v.n_slots + 255) / 256;
  const unsigned grid = (unsigned)(work < 1 ? 1 : (work < 65535 ? work : 65535));
  hipLaunchKernelGGL(validate_kernel, dim3(grid), dim3(256), 0, s, v);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(out, HIP_SYMBOL(g_kvs_check), 4 * sizeof(int), 0, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace kvs
